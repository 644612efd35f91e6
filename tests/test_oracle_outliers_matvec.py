"""Pins of the oracle's outlier selection/split and of the float64 product it
takes as the reference for every GPU result."""

from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synthetic
from conftest import load_golden


def test_outlier_counts():
    g = load_golden("otf_outlier_counts.json")
    for K, n in g["counts"].items():
        assert O.outlier_count(int(K), g["ratio"]) == n


def test_selection_matches_brute_force():
    """I_c = ||W[:, c]||_2 * profile_c (OTF section 4), top floor(0.035 K)."""
    rng = np.random.default_rng(21)
    N, K = 300, 1024
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    prof = np.abs(rng.standard_normal(K))
    idx = O.select_outliers(W, prof, 0.035)
    score = np.linalg.norm(W.astype(np.float64), axis=0) * prof
    order = np.argsort(-score, kind="stable")
    n = int(0.035 * K)
    assert score[order[n - 1]] - score[order[n]] > 1e-9 * score.max()   # no near-tie at the cut
    assert idx.dtype == np.int32 and np.all(np.diff(idx) > 0)
    assert set(idx.tolist()) == set(order[:n].tolist())


def test_selection_ties_go_to_lower_index():
    rng = np.random.default_rng(22)
    W = rng.standard_normal((16, 64), dtype=np.float32) * np.float32(0.01)
    W[:, 10] = W[:, 50] = 1.0          # equal columns, equal profile -> exact tie
    W[:, 20] = 2.0                     # clear winner
    prof = np.ones(64)
    idx = O.select_outliers(W, prof, 2 / 64 + 1e-9)
    assert idx.tolist() == [10, 20]


def test_spiked_channels_are_selected():
    """A profile with 1% of channels x100 (the 14336x4096 W2 workload's recipe,
    scaled down) puts every spiked channel in the outlier set."""
    L = synthetic.small_layer(2, 256, 4096, with_outliers=True, seed=3)
    idx = O.select_outliers(L.W, L.profile, L.ratio)
    assert len(idx) == 143 and set(L.spikes.tolist()) <= set(idx.tolist())


def test_split():
    rng = np.random.default_rng(23)
    W = rng.standard_normal((8, 96), dtype=np.float32)
    idx = np.array([0, 31, 32, 95], np.int32)
    dense, wout = O.split_outliers(W, idx)
    assert np.all(dense[:, idx] == 0)
    keep = np.setdiff1d(np.arange(96), idx)
    assert np.array_equal(dense[:, keep], W[:, keep])
    assert wout.dtype == np.float16 and wout.shape == (8, 4)
    assert np.array_equal(wout, W[:, idx].astype(np.float16))


def _exact_rows(w_hat, x, idx, wout):
    """Exact rational value of the fused product, term by term."""
    M, K = x.shape
    N = w_hat.shape[0]
    mask = O.background_mask(K, idx) if idx is not None else np.ones(K, bool)
    out = np.zeros((M, N))
    for m in range(M):
        xs = [Fraction(float(v)) for v in x[m].astype(np.float64)]
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                if mask[k]:
                    acc += Fraction(float(w_hat[n, k])) * xs[k]
            if idx is not None:
                for j, c in enumerate(idx):
                    acc += Fraction(float(wout[n, j])) * xs[int(c)]
            out[m, n] = float(acc)
    return out


@pytest.mark.parametrize("fmt", [4, 2])
def test_matvec_ref_against_exact_rationals(fmt):
    """64x64 brute force: the float64 reference equals the exact rational sums."""
    L = synthetic.small_layer(fmt, 64, 64, M=2, with_outliers=True, seed=fmt, ratio=0.07)
    Q = O.quantize_layer(fmt, L.W, L.profile, L.ratio)
    assert Q.n_out == 4
    y, a = O.matvec_ref(Q.w_hat(), L.x, Q.idx, Q.wout)
    ex = _exact_rows(Q.w_hat(), L.x, Q.idx, Q.wout)
    assert np.all(np.abs(y - ex) <= 1e-12 * a + 1e-300)
    # without outliers
    y0, a0 = O.matvec_ref(Q.w_hat(), L.x)
    ex0 = _exact_rows(Q.w_hat(), L.x, None, None)
    assert np.all(np.abs(y0 - ex0) <= 1e-12 * a0 + 1e-300)


def test_tolerance_check_behaviour():
    L = synthetic.small_layer(4, 128, 512, M=3)
    Q = O.quantize_layer(4, L.W)
    y, a = O.matvec_ref(Q.w_hat(), L.x)
    # an FP16-rounded exact answer is always inside the bound (2^-11 < 2e-3)
    ok, worst = O.check_tolerance(y.astype(np.float16), y, a)
    assert ok and worst < 0.3
    bad = y.copy()
    bad[1, 7] += 3 * (O.TOL_REL * a[1, 7] + O.TOL_ABS)
    assert not O.check_tolerance(bad, y, a)[0]
    nan = y.copy()
    nan[0, 0] = np.nan
    assert not O.check_tolerance(nan, y, a)[0]


def test_fp16_conversion_is_round_to_nearest_even():
    """The oracle relies on numpy's float64/float32 -> float16 casts being
    round-to-nearest-even: check at exact midpoints between FP16 neighbours."""
    h = np.arange(0x0001, 0x7BFF, dtype=np.uint16).view(np.float16)
    lo = h[:-1].astype(np.float64)
    hi = h[1:].astype(np.float64)
    mid = (lo + hi) / 2
    r = mid.astype(np.float16).view(np.uint16)
    even = np.where(h[:-1].view(np.uint16) % 2 == 0, h[:-1].view(np.uint16), h[1:].view(np.uint16))
    assert np.array_equal(r, even)
    r32 = mid.astype(np.float32).astype(np.float16).view(np.uint16)   # midpoints are exact in fp32
    assert np.array_equal(r32, even)
