"""Pins of the oracle's W2 quantizer (Lloyd-Max codes + OLS scale/zero), packer
and dequantizer against the OTF-LLM v4.0 page and the mathematics it states."""

import numpy as np
import pytest
from scipy import integrate, stats

import oracle as O
from conftest import load_golden


def test_codebook_matches_page():
    g = load_golden("otf_codebook.json")
    assert list(O.CODEBOOK_DECIMAL) == g["codebook"]
    hexes = [format(int(v), "04x") for v in O.CODEBOOK_FP16.view(np.uint16)]
    assert hexes == g["fp16_hex"]


def _gauss_mse(levels, thresholds):
    """Mean squared error of a scalar quantizer on N(0,1), by quadrature."""
    edges = np.concatenate([[-np.inf], thresholds, [np.inf]])
    tot = 0.0
    for c, a, b in zip(levels, edges[:-1], edges[1:]):
        tot += integrate.quad(lambda t: (t - c) ** 2 * stats.norm.pdf(t), a, b)[0]
    return tot


def _lloyd_step(levels):
    th = (levels[:-1] + levels[1:]) / 2
    edges = np.concatenate([[-np.inf], th, [np.inf]])
    new = []
    for a, b in zip(edges[:-1], edges[1:]):
        mass = stats.norm.cdf(b) - stats.norm.cdf(a)
        mean = (stats.norm.pdf(a) - stats.norm.pdf(b)) / mass     # E[t | a < t < b]
        new.append(mean)
    return np.array(new)


def test_codebook_is_lloyd_max_for_gaussian():
    """OTF section 2: the codebook minimises the quantization MSE of a normal
    distribution.  Checked by the Lloyd conditions (centroid = conditional mean
    of its cell, thresholds = midpoints), computed by quadrature."""
    cb = O.CODEBOOK_F64
    step = _lloyd_step(cb)
    assert np.max(np.abs(step - cb)) < 0.015            # codebook ~ a fixed point
    lv = cb.copy()
    for _ in range(200):
        lv = _lloyd_step(lv)
    assert np.max(np.abs(lv - cb)) < 0.012               # converged optimum ~ +-0.453, +-1.510
    mse_cb = _gauss_mse(cb, O.THRESHOLDS_F64)
    mse_opt = _gauss_mse(lv, (lv[:-1] + lv[1:]) / 2)
    assert abs(mse_cb - 0.1175) < 5e-4 and mse_cb / mse_opt - 1 < 1e-3
    for i in range(4):
        for d in (-0.05, 0.05):
            p = cb.copy()
            p[i] += d
            assert _gauss_mse(p, (p[:-1] + p[1:]) / 2) > mse_cb


def test_ols_equals_least_squares_solution():
    """OTF section 3: (S, Z) is the closed-form least-squares fit of w on the
    assigned centroids; compare with numpy's lstsq of [c, 1] against w."""
    rng = np.random.default_rng(5)
    W = rng.standard_normal((64, 256), dtype=np.float32) * np.float32(0.02)
    W += np.repeat(rng.standard_normal((64, 8), dtype=np.float32) * np.float32(0.005), 32, axis=1)
    q, S_h, Z_h, S, Z = O.quantize_w2(W, return_unrounded=True)
    c = O.CODEBOOK_F64[q.reshape(64, 8, 32)]
    Wg = W.reshape(64, 8, 32).astype(np.float64)
    worst = 0.0
    for i in range(64):
        for j in range(8):
            A = np.stack([c[i, j], np.ones(32)], axis=1)
            (s_ls, z_ls), *_ = np.linalg.lstsq(A, Wg[i, j], rcond=None)
            scale = abs(s_ls) + abs(z_ls)
            worst = max(worst, abs(S[i, j] - s_ls) / scale, abs(Z[i, j] - z_ls) / scale)
    assert worst < 1e-9
    assert np.array_equal(S_h, S.astype(np.float16)) and np.array_equal(Z_h, Z.astype(np.float16))


def test_ols_is_a_minimum():
    rng = np.random.default_rng(6)
    W = rng.standard_normal((16, 64), dtype=np.float32)
    q, _, _, S, Z = O.quantize_w2(W, return_unrounded=True)
    c = O.CODEBOOK_F64[q.reshape(16, 2, 32)]
    Wg = W.reshape(16, 2, 32).astype(np.float64)

    def sse(s, z):
        return ((Wg - (s[..., None] * c + z[..., None])) ** 2).sum(axis=2)

    base = sse(S, Z)
    for ds, dz in ((1e-3, 0), (-1e-3, 0), (0, 1e-3), (0, -1e-3)):
        assert np.all(sse(S + ds, Z + dz) > base)


def test_assignment_is_nearest_centroid():
    """The code of each weight is the nearest FP16 centroid to its standardised
    value (the reading of the unstated assignment step); ties go to the lower code."""
    rng = np.random.default_rng(8)
    W = rng.standard_normal((128, 512), dtype=np.float32)
    q, _, _ = O.quantize_w2(W)
    Wg = W.reshape(128, 16, 32).astype(np.float64)
    u = (Wg - Wg.mean(axis=2, keepdims=True)) / Wg.std(axis=2, keepdims=True)
    dist = np.abs(u[..., None] - O.CODEBOOK_F64)            # [.., 32, 4]
    brute = np.argmin(dist, axis=-1)                          # first minimum = lower code
    near_tie = np.min(np.abs(u[..., None] - O.THRESHOLDS_F64), axis=-1) < 1e-9
    agree = brute == q.reshape(128, 16, 32)
    assert np.all(agree | near_tie)
    # an exact tie goes to the lower code: a weight equal to its group mean has
    # u = 0, equidistant from -0.45 and +0.45 -> code 1
    grp = np.array([-1.0] * 15 + [0.0, 0.0] + [1.0] * 15, np.float32)
    qt = O.quantize_w2(grp[None, :])[0][0]
    assert qt[15] == 1 and qt[16] == 1 and set(qt[:15].tolist()) == {0} and set(qt[17:].tolist()) == {3}


def test_code_histogram_on_gaussian_groups():
    """Nearest-centroid codes of Gaussian groups fall into the outer cells with
    probability close to Phi(-0.9847) = 0.162 (slightly more after
    standardising by each group's own mean and spread)."""
    rng = np.random.default_rng(9)
    W = rng.standard_normal((1024, 1024), dtype=np.float32)
    q, _, _ = O.quantize_w2(W)
    h = np.bincount(q.ravel(), minlength=4) / q.size
    outer = stats.norm.cdf(O.THRESHOLDS_F64[0])
    assert abs(outer - 0.1624) < 1e-3
    for i, p in enumerate((outer, 0.5 - outer, 0.5 - outer, outer)):
        assert abs(h[i] - p) < 0.006


def test_special_groups():
    g = np.zeros((2, 32), np.float32)
    g[0] = 0.125                                 # zero variance
    g[1, ::2], g[1, 1::2] = -0.5, 0.5            # two values
    q, S, Z, S64, Z64 = O.quantize_w2(g, return_unrounded=True)
    assert np.all(q[0] == 1) and S64[0, 0] == 0.0 and Z64[0, 0] == 0.125
    assert np.all(O.dequant_w2(q, S, Z)[0] == np.float16(0.125))
    # two-valued group: standardised to +-1 -> codes 0/3 (|u| = 1 > 0.9847)
    assert set(q[1].tolist()) == {0, 3}


def test_dequant_hand_values():
    q = np.tile(np.arange(4, dtype=np.uint8), 8)[None, :]
    one = np.array([[1.0]], np.float16)
    zero = np.array([[0.0]], np.float16)
    assert np.array_equal(O.dequant_w2(q, one, zero)[0], np.tile(O.CODEBOOK_FP16, 8))
    # S = 2, Z = 0.5: exact in FP16 -> 2c + 0.5 rounded once
    two, half = np.array([[2.0]], np.float16), np.array([[0.5]], np.float16)
    exp = (2.0 * O.CODEBOOK_FP16.astype(np.float64) + 0.5).astype(np.float16)
    assert np.array_equal(O.dequant_w2(q, two, half)[0], np.tile(exp, 8))


def test_pack_exhaustive_roundtrip():
    b = np.arange(256, dtype=np.uint8)[None, :]
    q = O.unpack_w2(b)
    assert q.shape == (1, 1024) and q.max() <= 3
    assert np.array_equal(O.pack_w2(q), b)
    rng = np.random.default_rng(1)
    qr = rng.integers(0, 4, (17, 128), dtype=np.uint8)
    assert np.array_equal(O.unpack_w2(O.pack_w2(qr)), qr)


def test_pack_hand_example():
    g = load_golden("w2_pack_example.json")
    q = np.array(g["codes"], np.uint8)[None, :]
    assert O.pack_w2(q)[0].tobytes().hex() == g["bytes_hex"]


def test_background_must_skip_outlier_columns():
    """Zeroed outlier columns do not reconstruct to 0 under W2 (S*c + Z != 0),
    so the quantized background has to skip them; without the mask the error
    grows with the spike."""
    rng = np.random.default_rng(12)
    N, K = 64, 256
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    prof = np.ones(K)
    prof[[3, 77]] = 100.0
    L = O.quantize_layer(2, W, prof, 0.035)
    w_hat = L.w_hat().astype(np.float64)
    assert np.any(w_hat[:, L.idx] != 0)
    x = rng.standard_normal((1, K)).astype(np.float16)
    errs = []
    for mult in (1.0, 300.0):
        xm = x.astype(np.float32)
        xm[0, [3, 77]] *= mult
        xm = xm.astype(np.float16)
        y, _ = O.matvec_ref(L.w_hat(), xm, L.idx, L.wout)
        y_nomask = xm.astype(np.float64) @ w_hat.T + xm.astype(np.float64)[:, L.idx] @ L.wout.astype(np.float64).T
        exact = xm.astype(np.float64) @ W.astype(np.float64).T
        errs.append((np.abs(y - exact).max(), np.abs(y_nomask - exact).max()))
    assert errs[1][1] > 10 * errs[1][0]          # unmasked background is far worse
    assert errs[1][1] > 10 * errs[0][1]          # and its error grows with the spike
