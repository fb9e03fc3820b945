"""Statistical acceptance rules used by the sampling-law tests (test infrastructure).

The rules are the ones the Megatron-LM "fp64 sampling noise" pull request states
in its "Tests" section, made precise:

* tail rate: the number of draws that miss token 0 of a row [0, -D, ..., -D]
  with V entries must lie in the two-sided 1e-6 Poisson interval of the exact
  rate.  Under softmax the miss probability is q = (V-1) r / (1 + (V-1) r) with
  r = e^-D (the "Problem" section); the interval accepts a count c iff
  P(X <= c) > 5e-7 and P(X >= c) > 5e-7 for X ~ Poisson(N q).
* chi-square: over a 16-token row, the statistic must stay below the 1e-6
  upper quantile of chi-square with 15 degrees of freedom (the page rounds it
  to 56.5).
"""
from __future__ import annotations

import numpy as np
from scipy import stats


def miss_probability(V: int, D: float) -> float:
    """Exact softmax probability of not drawing token 0 from [0, -D, ..., -D]."""
    r = np.exp(-np.float64(D))
    return float((V - 1) * r / (1.0 + (V - 1) * r))


def poisson_two_sided_ok(count: int, lam: float, alpha: float = 1e-6) -> bool:
    """True iff count lies in the two-sided `alpha` Poisson interval of mean lam."""
    lo_tail = stats.poisson.cdf(count, lam)          # P(X <= count)
    hi_tail = stats.poisson.sf(count - 1, lam)       # P(X >= count)
    return bool(lo_tail > alpha / 2 and hi_tail > alpha / 2)


def poisson_interval(lam: float, alpha: float = 1e-6):
    """Smallest and largest accepted counts under poisson_two_sided_ok."""
    lo = int(stats.poisson.ppf(alpha / 2, lam))
    while lo > 0 and poisson_two_sided_ok(lo - 1, lam, alpha):
        lo -= 1
    while not poisson_two_sided_ok(lo, lam, alpha):
        lo += 1
    hi = int(stats.poisson.isf(alpha / 2, lam))
    while poisson_two_sided_ok(hi + 1, lam, alpha):
        hi += 1
    while not poisson_two_sided_ok(hi, lam, alpha):
        hi -= 1
    return lo, hi


def chi2_quantile(dof: int, alpha: float = 1e-6) -> float:
    return float(stats.chi2.isf(alpha, dof))


def chi2_statistic(counts: np.ndarray, probs: np.ndarray) -> float:
    counts = np.asarray(counts, dtype=np.float64)
    expected = counts.sum() * np.asarray(probs, dtype=np.float64)
    assert np.all(expected >= 5.0), "chi-square needs every expected count >= 5"
    return float(((counts - expected) ** 2 / expected).sum())


def softmax64(y) -> np.ndarray:
    y = np.asarray(y, dtype=np.float64)
    m = np.max(y[np.isfinite(y)])
    e = np.where(np.isfinite(y), np.exp(y - m), 0.0)
    return e / e.sum()
