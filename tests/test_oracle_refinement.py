"""Pins of the oracle's runtime top-k refinement (StrataFlux page, section
3.2.1, "Channel selection" and Eq. 2): the selection against brute-force
sorting and hand-worked cases (ties, signs, short last chunk, k at least the
chunk), the refinement columns against the pinned W4 quantizer, and the
refined product against exact rational arithmetic."""

from fractions import Fraction

import numpy as np
import pytest

import oracle as O


def brute_topk(x, k, chunk):
    x = np.asarray(x, np.float16)
    out = []
    for c0 in range(0, len(x), chunk):
        items = [(-abs(float(x[i])), i) for i in range(c0, min(c0 + chunk, len(x)))]
        items.sort()
        out += sorted(i for _, i in items[:k])
    return out


def test_topk_hand_example():
    # chunk of 4: |x| = 3, 1, 3, 0.5 and 2, 2, 5, 0 -> k = 2 picks {0, 2} (the tie of
    # the two 3s keeps both), then {6} plus the lower index of the tied 2s, {4}
    x = np.array([3.0, -1.0, -3.0, 0.5, 2.0, -2.0, -5.0, 0.0], np.float16)
    assert O.topk_chunks(x, 2, chunk=4).tolist() == [0, 2, 4, 6]
    # a short last chunk gives all it has; k >= chunk takes every channel
    assert O.topk_chunks(x[:6], 3, chunk=4).tolist() == [0, 1, 2, 4, 5]
    assert O.topk_chunks(x, 9, chunk=4).tolist() == list(range(8))
    assert O.topk_chunks(x, 0, chunk=4).tolist() == []


@pytest.mark.parametrize("K,k,chunk", [(4096, 32, 1024), (14336, 32, 1024), (1000, 7, 64),
                                       (3000, 1, 1024), (2048, 1024, 1024)])
def test_topk_matches_brute_force(K, k, chunk):
    rng = np.random.default_rng(K + k)
    x = rng.standard_normal(K).astype(np.float16)
    x[rng.choice(K, K // 10)] = x[0]            # many exact ties
    x[::97] *= -50                              # large negative values
    assert O.topk_chunks(x, k, chunk).tolist() == brute_topk(x, k, chunk)


def test_refinement_columns_are_w4_of_the_residual():
    rng = np.random.default_rng(4)
    W = (0.02 * rng.standard_normal((64, 96))).astype(np.float32)
    q, sc, ze, _ = O.quantize_w4(W)
    w_hat = O.dequant_w4(q, sc, ze)
    rq, rs, rz = O.refinement_w4(W, w_hat)
    assert rq.shape == (96, 64) and rs.shape == (96, 2)
    R = W - w_hat.astype(np.float32)
    c_hat = O.dequant_w4(rq, rs, rz).astype(np.float64)
    # the refined weights are closer to W than the resident ones, column by column
    err0 = np.abs(R).max(axis=0)
    err1 = np.abs(R.T - c_hat).max(axis=1)
    assert np.all(err1 <= err0 / 2 + 1e-7)
    # each refinement value within half a step of the residual (SPECTRA Prop. 2
    # on R^T), apart from the FP16 rounding of the scale (|q - z| <= 15 steps,
    # each off by at most 2^-11 of a step) and of the value itself
    step = rs.astype(np.float64).repeat(32, axis=1)
    bound = step / 2 + 15 * step * 2.0**-11 + np.abs(c_hat) * 2.0**-11 + 1e-12
    assert np.all(np.abs(R.T - c_hat) <= bound)


def test_refine_ref_exact_rationals():
    rng = np.random.default_rng(5)
    N, K = 48, 64
    C = rng.standard_normal((K, N)).astype(np.float16)
    x = rng.standard_normal(K).astype(np.float16)
    y0 = rng.standard_normal(N).astype(np.float16)
    sel = O.topk_chunks(x, 5, chunk=16)
    y, a = O.refine_ref(y0, x, sel, C)
    for n in range(N):
        exact = Fraction(float(y0[n])) + sum(Fraction(float(x[i])) * Fraction(float(C[i, n]))
                                             for i in sel)
        assert abs(Fraction(y[n]) - exact) <= Fraction(1, 10**12) * (1 + abs(exact))
        assert a[n] >= abs(float(exact)) * (1 - 1e-12)


def _hand_layer():
    """A 32 x 64 layer whose residual the W4 grid holds exactly: with w_hat = 0
    the residual is W itself, W[n, c] = ((n + c) mod 16) / 8.  Each refinement
    group (32 output rows of one input channel) then spans 0 .. 15/8, so
    s = (15/8) / 15 = 1/8 exactly, z = 0 and q = (n + c) mod 16: the dequantized
    refinement equals W^T bit for bit."""
    n = np.arange(32)[:, None]
    c = np.arange(64)[None, :]
    W = (((n + c) % 16) / 8.0).astype(np.float32)
    return W, np.zeros((32, 64), np.float16)


def _refined_rows(fn, W, w_hat, idx):
    q, s, z = fn(W, w_hat, idx)
    return O.dequant_w4(q, s, z).astype(np.float64)


def _idx_branch_holds(fn):
    """StrataFlux section 3.2.1 with the resident layer's outlier columns Omega
    (held exactly in FP16): their residual is 0.  Omega lies below N = 32, so
    that applying it to the output rows instead is a valid (wrong) index.  Per input channel c of R^T:
    c in Omega -> the dequantized refinement row is exactly 0; every other
    channel's row equals the one computed without Omega (refinement groups run
    along N inside one channel, so zeroing one channel cannot move another)."""
    W, w_hat = _hand_layer()
    idx = np.array([3, 17, 29], np.int32)
    with_idx = _refined_rows(fn, W, w_hat, idx)
    without = _refined_rows(fn, W, w_hat, None)
    others = np.setdiff1d(np.arange(64), idx)
    return (with_idx.shape == (64, 32)
            and np.all(with_idx[idx] == 0.0)
            and np.array_equal(with_idx[others], without[others])
            and np.array_equal(without, W.T.astype(np.float64)))


def test_refinement_outlier_columns_hand_worked():
    W, w_hat = _hand_layer()
    idx = np.array([3, 17, 29], np.int32)
    c_hat = _refined_rows(O.refinement_w4, W, w_hat, idx)
    expect = W.T.astype(np.float64).copy()
    expect[idx] = 0.0
    assert np.array_equal(c_hat, expect)
    # the zeroed channels encode as an all-zero group: codes 0, zero point 0,
    # and the 1e-8 scale floor, which FP16 rounds to 0
    q, s, z = O.refinement_w4(W, w_hat, idx)
    assert np.all(q[idx] == 0) and np.all(z[idx] == 0) and np.all(s[idx] == 0)
    assert _idx_branch_holds(O.refinement_w4)


def test_refinement_outlier_branch_catches_rows_for_columns():
    # a planted mistake in the oracle's branch: the outlier set applied to the
    # output rows of R (R[idx, :]) instead of its input channels
    def rows_instead(W, w_hat, idx=None):
        R = np.asarray(W, np.float32) - np.asarray(w_hat, np.float16).astype(np.float32)
        if idx is not None and len(idx):
            R[np.asarray(idx, np.int64), :] = 0.0
        q, sc, ze, _ = O.quantize_w4(np.ascontiguousarray(R.T))
        return q, sc, ze

    # and one that forgets the branch altogether
    def no_branch(W, w_hat, idx=None):
        return O.refinement_w4(W, w_hat, None)

    assert not _idx_branch_holds(rows_instead)
    assert not _idx_branch_holds(no_branch)
