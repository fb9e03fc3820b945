"""Values the pages print, checked against the closed forms the tests rely on.

Megatron-LM "fp64 sampling noise" page: the tail table ("Problem") prints the
expected miss counts and the two-sided Poisson p-values of the observed counts;
"Tests" prints the chi-square threshold 56.5 (1e-6, 15 dof) and the float32
non-vacuity expectation 34 at r = 1e-9 over 262k draws of V = 131072.
"""
import numpy as np
import pytest
from scipy import stats

import synthetic
from conftest import read_golden
from oracle import stats as st


def _table():
    rows = read_golden("megatron_tail_table.txt")
    V = int(rows[0][1])
    return V, [[float(x) for x in r] for r in rows[1:]]


def test_expected_tail_counts_match_closed_form():
    V, rows = _table()
    for r, draws, expected, *_ in rows:
        lam = draws * st.miss_probability(V, synthetic.tail_depth(r))
        # the page's draw counts are rounded; its expected counts sit 0.3-0.7% above
        assert lam == pytest.approx(expected, rel=0.01), (r, lam, expected)


def _two_sided_p(c, lam):
    return min(1.0, 2 * min(stats.poisson.cdf(c, lam), stats.poisson.sf(c - 1, lam)))


def test_printed_p_values_reproduce():
    V, rows = _table()
    for r, draws, expected, fp64_obs, fp64_p, torch_obs, torch_p in rows:
        assert _two_sided_p(int(fp64_obs), expected) == pytest.approx(fp64_p, abs=0.03)
        if not np.isnan(torch_p):
            p = _two_sided_p(int(torch_obs), expected)
            assert np.log10(p) == pytest.approx(np.log10(torch_p), abs=1.0)


def test_fp64_counts_accepted_fp32_tail_counts_rejected():
    """The page's fp64 column passes the 1e-6 interval; the starved float32
    counts at r <= 1e-8 fail it."""
    V, rows = _table()
    for r, draws, expected, fp64_obs, _, torch_obs, _ in rows:
        assert st.poisson_two_sided_ok(int(fp64_obs), expected)
        if r <= 1e-8:
            assert not st.poisson_two_sided_ok(int(torch_obs), expected)


def test_chi2_threshold_and_nonvacuity_expectation():
    facts = {k: float(v) for k, v in read_golden("megatron_noise_facts.txt")}
    assert round(st.chi2_quantile(int(facts["chi2_dof"])), 1) == facts["chi2_q1e6"]
    lam = facts["tail_draws"] * st.miss_probability(int(facts["tail_V"]),
                                                    synthetic.tail_depth(1e-9))
    assert round(lam) == facts["nonvacuity_expected"]
    lo, hi = st.poisson_interval(lam)
    assert lo > 0          # so an observed 0 is a rejection
