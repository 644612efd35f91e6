"""Pins of the oracle's kurtosis-adaptive outlier policy (SPECTRA page,
sections 3.1-3.3 and Appendix A Proposition 1): the ratio rule at the values
the page states, its closed form, Proposition 1's bound and its extreme case,
the kurtosis against an independent library routine and exact rational
arithmetic, and the selection on matrices whose answer is known."""

from fractions import Fraction

import numpy as np
import pytest

import oracle as O


def test_ratio_rule_page_values_and_closed_form():
    # mesokurtic saliencies keep r = r_base = 0.01 (section 3.3)
    for kappa in (0.0, 1.0, 2.999, 3.0):
        assert O.kurtosis_ratio(kappa) == 0.01
    # r_base (1 + 0.15 k) when kappa - 3 = e^k - 1
    for k in (0.5, 1.0, 2.0, 5.0):
        assert O.kurtosis_ratio(3.0 + np.expm1(k)) == pytest.approx(0.01 * (1 + 0.15 * k), rel=1e-12)
    # the strict 3% cap: reached once 0.15 ln(1 + excess) >= 2
    edge = np.expm1(2.0 / 0.15)
    assert O.kurtosis_ratio(3.0 + edge * 1.001) == 0.03
    assert O.kurtosis_ratio(3.0 + edge * 0.99) < 0.03
    assert O.kurtosis_ratio(1e12) == 0.03
    # the lower clamp never binds at r_base = 0.01, but does for a smaller base
    assert O.kurtosis_ratio(3.0, r_base=0.001) == 0.005


def test_kurtosis_hand_example_exact():
    S = [1, 2, 3, 4, 10]
    K = len(S)
    mu = Fraction(sum(S), K)
    var = sum((Fraction(v) - mu) ** 2 for v in S) / K
    kappa = sum((Fraction(v) - mu) ** 4 for v in S) / K / (var * var)
    assert O.saliency_kurtosis(np.array(S, float)) == pytest.approx(float(kappa), rel=1e-14)


def test_kurtosis_matches_library_routine():
    stats = pytest.importorskip("scipy.stats")
    rng = np.random.default_rng(7)
    for S in (rng.standard_normal(4096), np.abs(rng.standard_cauchy(2048)),
              rng.exponential(size=999), rng.uniform(size=50)):
        ref = stats.kurtosis(S, fisher=False, bias=True)   # population fourth standardized moment
        assert O.saliency_kurtosis(S) == pytest.approx(ref, rel=1e-12)


def test_proposition1_bound_and_extreme_case():
    rng = np.random.default_rng(8)
    for K in (2, 5, 64, 4096):
        for S in (rng.standard_normal(K), np.abs(rng.standard_cauchy(K)) ** 3,
                  rng.exponential(size=K) ** 4):
            assert O.saliency_kurtosis(S) <= K * (1 + 1e-12)
        # one spike among equal values: kappa = ((K - 1)^2 + 1 / (K - 1)) / K, within 2 of K
        S = np.zeros(K)
        S[K // 3] = 7.0
        exact = ((K - 1) ** 2 + 1 / (K - 1)) / K
        assert O.saliency_kurtosis(S) == pytest.approx(exact, rel=1e-12)
        assert K - 2 <= exact <= K
    # Gaussian saliencies are mesokurtic: kappa -> 3
    assert O.saliency_kurtosis(np.random.default_rng(9).standard_normal(1_000_000)) == \
        pytest.approx(3.0, abs=0.02)
    assert O.saliency_kurtosis(np.full(10, 2.5)) == 0.0   # no spread (reading)


def test_selection_on_known_matrices():
    rng = np.random.default_rng(10)
    N, K = 64, 4096
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    # Gaussian columns: near-equal norms, mesokurtic, r = 1% -> floor(0.01 K) = 40 columns
    idx, r, kappa = O.select_outliers_kurtosis(W)
    assert kappa < 3.5 and r == pytest.approx(0.01 * (1 + 0.15 * np.log1p(max(0, kappa - 3))))
    assert len(idx) == int(np.floor(r * K)) and np.all(np.diff(idx) > 0)
    # the selected columns are the largest norms (brute force)
    norms = np.sqrt((W.astype(np.float64) ** 2).sum(axis=0))
    assert set(idx.tolist()) == set(np.argsort(-norms, kind="stable")[:len(idx)].tolist())
    # 41 heavy columns (x30): leptokurtic saliencies, r grows; every heavy column is selected
    heavy = rng.choice(K, 41, replace=False)
    W2 = W.copy()
    W2[:, heavy] *= 30.0
    idx2, r2, kappa2 = O.select_outliers_kurtosis(W2)
    assert kappa2 > 50 and r2 > r
    assert set(heavy.tolist()) <= set(idx2.tolist())
    # gamma weights the saliency: a gain of 100 on 5 columns puts them in the set
    gamma = np.ones(K)
    pick = np.array([3, 700, 1500, 2222, 4095])
    gamma[pick] = 100.0
    idx3, _, _ = O.select_outliers_kurtosis(W, gamma)
    assert set(pick.tolist()) <= set(idx3.tolist())
