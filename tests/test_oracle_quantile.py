"""Pins of the oracle's quantile clip threshold (oracle/quantile.py)."""
import numpy as np
import pytest

from oracle import quantile as QT


def test_matches_sorting_on_tiny_inputs():
    rng = np.random.default_rng(0)
    for n in (1, 2, 5, 16, 37, 100):
        x = rng.standard_normal(n).astype(np.float32)
        srt = np.sort(np.abs(x))                       # brute force
        for q in (0.01, 0.5, 0.9, 0.99, 1.0):
            k = int(np.ceil(q * n))
            assert QT.abs_quantile(x, q) == srt[max(k, 1) - 1]


def test_matches_numpy_inverted_cdf_quantile():
    # the inverted-CDF estimator is the library's method="inverted_cdf"
    rng = np.random.default_rng(1)
    x = (rng.standard_t(3, size=20000) * 0.02).astype(np.float32)
    for q in (0.5, 0.9, 0.99, 0.999):
        want = np.quantile(np.abs(x), q, method="inverted_cdf")
        assert QT.abs_quantile(x, q) == np.float32(want)


def test_order_statistic_counts():
    # at least ceil(qN) magnitudes at or below the threshold, fewer strictly below
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 48)).astype(np.float32)
    a = np.abs(x)
    for q in (0.25, 0.99):
        t = QT.abs_quantile(x, q)
        k = int(np.ceil(q * x.size))
        assert np.count_nonzero(a <= t) >= k
        assert np.count_nonzero(a < t) < k


def test_ties_signs_and_zeros():
    x = np.array([-3, 3, -3, 1, 0, -0.0, 2, -2], np.float32)   # |x| sorted: 0 0 1 2 2 3 3 3
    assert QT.abs_quantile(x, 0.25) == 0.0            # k = 2: the two zeros
    assert QT.abs_quantile(x, 0.375) == 1.0           # k = 3
    assert QT.abs_quantile(x, 0.5) == 2.0             # k = 4
    assert QT.abs_quantile(x, 0.75) == 3.0            # k = 6
    assert QT.abs_quantile(x, 1.0) == 3.0


def test_non_finite_sorts_last():
    x = np.ones(100, np.float32)
    x[:2] = [np.nan, -np.inf]
    assert QT.abs_quantile(x, 0.98) == 1.0            # k = 98 < 99
    assert np.isnan(QT.abs_quantile(x, 0.99))         # k = 99 reaches the non-finite


def test_rank_definition():
    assert QT.quantile_rank(0.99, 100) == 99
    assert QT.quantile_rank(1.0, 7) == 7
    assert QT.quantile_rank(1e-9, 7) == 1
    assert QT.quantile_rank(0.99, 25165824) == 24914166
    with pytest.raises(ValueError):
        QT.quantile_rank(0.0, 10)
