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
