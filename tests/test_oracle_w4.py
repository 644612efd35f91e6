"""Pins of the oracle's W4 quantizer, packer and dequantizer against what the
SPECTRA page fixes (printed values, propositions, hand-worked cases)."""

import numpy as np
import pytest

import oracle as O
from conftest import load_golden


def _recon_unrounded(q, zero, s):
    N, K = q.shape
    qg = q.reshape(N, K // 32, 32).astype(np.float64)
    return ((qg - zero.astype(np.float64)[..., None]) * s.astype(np.float64)[..., None]).reshape(N, K)


def test_experiment_a_gaussian_matrix():
    """SPECTRA section 5.7, Experiment A: 2048x2048 Gaussian, Group-32 ->
    8.08% relative error, 21.85 dB, cosine 0.99676, max error 0.50000 s."""
    g = load_golden("spectra_experiment_a.json")
    rng = np.random.default_rng(20260)
    W = rng.standard_normal((g["rows"], g["cols"]), dtype=np.float32)
    q, scale, zero, s = O.quantize_w4(W)
    w_hat = O.dequant_w4(q, scale, zero)
    rel, snr, cos = O.fidelity(W, w_hat)
    assert abs(100 * rel - g["rel_err_pct"]) < 0.05
    assert abs(snr - g["snr_db"]) < 0.05
    assert abs(cos - g["cosine"]) < 5e-5
    # Max error in units of the scale the codes were made with (Proposition 2
    # excludes the rounding of s to 16 bits).
    err = np.abs(W.astype(np.float64) - _recon_unrounded(q, zero, s))
    ratio = err.reshape(W.shape[0], -1, 32) / s.astype(np.float64)[..., None]
    m = float(ratio.max())
    assert g["max_err_over_scale"] - 1e-4 <= m <= 0.5 + 2e-6


def test_proposition2_bound_on_zero_spanning_groups():
    """|w - (q - z) s| <= s/2 whenever the group spans zero (SPECTRA Prop. 2)."""
    bound = load_golden("spectra_proposition2.json")["bound_in_units_of_s"]
    rng = np.random.default_rng(7)
    W = rng.standard_normal((256, 1024), dtype=np.float32) * np.float32(0.02)
    # add groups with a large offset that still straddle zero, and heavy tails
    W[:64] += np.float32(0.01)
    W[64:128] *= rng.standard_cauchy((64, 1024)).astype(np.float32)
    q, scale, zero, s = O.quantize_w4(W)
    Wg = W.reshape(256, 32, 32).astype(np.float64)
    spans = (Wg.min(axis=2) <= 0) & (Wg.max(axis=2) >= 0)
    assert spans.mean() > 0.9
    rec = _recon_unrounded(q, zero, s).reshape(Wg.shape)
    err = np.abs(Wg - rec) / s.astype(np.float64)[..., None]
    assert float(err[spans].max()) <= bound * (1 + 1e-5)


def test_proposition3_mean_range_and_prediction():
    """Mean range of 32 N(0,1) is d = 4.14, and the empirical error lies within
    0.11 pp of d / (15 sqrt 12) = 7.97% (SPECTRA Prop. 3)."""
    g = load_golden("spectra_proposition3.json")
    rng = np.random.default_rng(11)
    W = rng.standard_normal((4096, 1024), dtype=np.float32)   # 131072 groups
    q, scale, zero, s = O.quantize_w4(W)
    d = 15.0 * float(s.astype(np.float64).mean())
    assert abs(d - g["mean_range_d"]) < 0.01
    pred = d / (15.0 * np.sqrt(12.0))
    assert abs(100 * pred - g["rel_err_pct"]) < 0.02
    rel, snr, cos = O.fidelity(W, O.dequant_w4(q, scale, zero))
    assert 0.0 <= 100 * (rel - pred) <= g["max_gap_pct"] + 0.02
    assert 0.0 <= 20 * np.log10(15 * np.sqrt(12) / d) - snr <= g["max_gap_db"] + 0.02
    assert abs(cos - g["cosine"]) < 1.5e-4


def test_hand_worked_group_half_even():
    """A group whose arithmetic is exact in binary: range 3.75 -> s = 0.25,
    z = round(0.75 / 0.25) = 3; positions 16..30 sit exactly half-way between
    codes, so round-half-to-even decides them; position 31 repeats the minimum."""
    w = np.zeros(32, np.float32)
    w[:16] = -0.75 + 0.25 * np.arange(16)
    w[16:31] = -0.625 + 0.25 * np.arange(15)
    w[31] = -0.75
    q, scale, zero, s = O.quantize_w4(w[None, :])
    assert float(s[0, 0]) == 0.25 and float(scale[0, 0]) == 0.25
    assert float(zero[0, 0]) == 3.0
    expect = list(range(16)) + [0, 2, 2, 4, 4, 6, 6, 8, 8, 10, 10, 12, 12, 14, 14] + [0]
    assert q[0].tolist() == expect
    w_hat = O.dequant_w4(q, scale, zero)[0].astype(np.float64)
    assert np.array_equal(w_hat, (np.array(expect) - 3) * 0.25)


def test_special_groups():
    rows = np.zeros((4, 32), np.float32)
    rows[1] = 0.5                                   # constant, non-zero
    rows[2] = -np.linspace(1.0, 2.0, 32, dtype=np.float32)   # all negative
    rows[3] = np.linspace(1.0, 2.0, 32, dtype=np.float32)    # all positive
    q, scale, zero, s = O.quantize_w4(rows)
    # all-zero group: floor scale 1e-8, which FP16 rounds to 0 -> exact zeros
    assert float(s[0, 0]) == np.float32(1e-8) and float(scale[0, 0]) == 0.0
    assert np.all(q[0] == 0) and float(zero[0, 0]) == 0.0
    w_hat = O.dequant_w4(q, scale, zero)
    assert np.all(w_hat[0] == 0) and np.all(w_hat[1] == 0)
    # constant 0.5: -wmin/s < 0 clamps z to 0; every code saturates at 15
    assert float(zero[1, 0]) == 0.0 and np.all(q[1] == 15)
    # one-sided groups clamp the zero point at the ends of 0..15
    assert float(zero[2, 0]) == 15.0
    assert float(zero[3, 0]) == 0.0


def test_zeroed_columns_reconstruct_exactly_zero():
    """Columns zeroed by the outlier split reconstruct to exactly 0: a group that
    contains a 0 spans zero, so z is not clamped and round(0/s + z) = z."""
    rng = np.random.default_rng(3)
    W = rng.standard_normal((128, 512), dtype=np.float32) * np.float32(0.02)
    cols = rng.choice(512, 40, replace=False)
    for m in (1.0, 100.0, 1e4):
        Wm = W.copy()
        Wm[:, cols[:5]] *= np.float32(m)
        Wm[:, cols] = 0.0
        q, scale, zero, s = O.quantize_w4(Wm)
        w_hat = O.dequant_w4(q, scale, zero)
        assert np.all(w_hat[:, cols] == 0)


def test_pack_exhaustive_roundtrip():
    lo, hi = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    pairs = np.stack([lo.ravel(), hi.ravel()], axis=1)          # 256 (lo, hi)
    q = np.zeros((256, 32), np.uint8)
    q[:, 5] = pairs[:, 0]
    q[:, 21] = pairs[:, 1]
    codes = O.pack_w4(q)
    assert codes.shape == (256, 16)
    assert sorted(codes[:, 5].tolist()) == list(range(256))
    assert np.array_equal(O.unpack_w4(codes), q)
    rng = np.random.default_rng(0)
    qr = rng.integers(0, 16, (33, 96), dtype=np.uint8)
    assert np.array_equal(O.unpack_w4(O.pack_w4(qr)), qr)


def test_pack_hand_example():
    g = load_golden("w4_pack_example.json")
    q = np.array(g["codes"], np.uint8)[None, :]
    assert O.pack_w4(q)[0].tobytes().hex() == g["bytes_hex"]


# ------------------------------------------------------- packed zero points


def test_packed_zero_hand_example():
    g = load_golden("w4_packed_zero_example.json")
    z = np.array(g["zeros"], np.float16)[None, :]
    zpk = O.pack_zeros_w4(z)
    assert zpk[0].tobytes().hex() == g["bytes_hex"]
    assert np.array_equal(O.unpack_zeros_w4(zpk, z.shape[1]), z)


def test_packed_zero_exhaustive_roundtrip():
    # every byte value decodes to two zero points and packs back to itself
    b = np.arange(256, dtype=np.uint8)[:, None]
    z = O.unpack_zeros_w4(b, 2)
    assert sorted(set(z.ravel().tolist())) == list(range(16))
    assert np.array_equal(z[:, 0], (b[:, 0] & 15).astype(np.float16))
    assert np.array_equal(z[:, 1], (b[:, 0] >> 4).astype(np.float16))
    assert np.array_equal(O.pack_zeros_w4(z), b)


def test_packed_zero_layer_and_rejects():
    # the zero points the quantizer makes always pack, and packing loses nothing
    rng = np.random.default_rng(3)
    W = rng.standard_normal((9, 32 * 7)).astype(np.float32)
    W[:, :32] -= 5.0                 # an all-negative group: z clamps to 15
    W[:, 32:64] += 5.0               # an all-positive group: z = 0
    _, _, zero, _ = O.quantize_w4(W)
    zpk = O.pack_zeros_w4(zero)
    assert zpk.shape == (9, 4) and np.all(zpk[:, 3] >> 4 == 0)
    assert np.array_equal(O.unpack_zeros_w4(zpk, 7), zero)
    assert np.all(zero[:, 0] == 15) and np.all(zero[:, 1] == 0)
    for bad in (np.array([[16.0]]), np.array([[-1.0]]), np.array([[2.5]])):
        with pytest.raises(ValueError):
            O.pack_zeros_w4(bad.astype(np.float16))
