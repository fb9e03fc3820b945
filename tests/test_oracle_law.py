"""Pin the law of the oracle's sampler to softmax.

* Gumbel-max over the noise grid equals softmax sampling (FlashSampling page,
  prerequisites: the argmax of logits plus Gumbel noise is a sample from
  softmax).  Checked by exact enumeration of the 2^23-point float32 noise grid for
  two- and three-token rows, independently of the oracle, and by the oracle's own
  draws against that exact law.
* Chi-square over a 16-token row, 1M draws, below the 1e-6 quantile with 15 dof
  (Megatron-LM "fp64 sampling noise" page, section "Tests"), for both noise
  widths and for the fused path with bias and temperature.
* Tail rate: misses of token 0 of [0, -D, ..., -D] inside the two-sided 1e-6
  Poisson interval of the exact miss probability (same page, "Problem" and
  "Tests").  A moderate depth runs by default; the page's depth runs under
  FS_SLOW=1.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from oracle import stats as st


def _grid_gumbel(bits=23):
    """g for every point of the midpoint grid, increasing in u (numpy, not the oracle)."""
    k = np.arange(2**bits, dtype=np.float64)
    u = (k + 0.5) / 2.0**bits
    E = np.where(u >= 0.5, -np.log1p(u - 1.0), -np.log(u))
    return -np.log(E)


def _exact_grid_law(y, G):
    """P(token k) for argmax_i (y_i + g_i), g iid on grid G, smaller index wins ties."""
    n = len(G)
    y = np.asarray(y, dtype=np.float64)
    P = np.zeros(len(y))
    for k in range(len(y)):
        prob = np.ones(n)
        for j in range(len(y)):
            if j == k:
                continue
            thr = G + y[k] - y[j]              # need g_j < thr (j < k) or <= thr (j > k)
            side = "left" if j < k else "right"
            prob *= np.searchsorted(G, thr, side=side) / n
        P[k] = prob.mean()
    return P


@pytest.fixture(scope="module")
def G23():
    G = _grid_gumbel(23)
    assert np.all(np.diff(G) > 0)
    return G


def test_grid_law_equals_softmax(G23):
    for y in ([0.0, -1.0], [1.3, -0.4, 0.2], [0.0, -8.0]):
        P = _exact_grid_law(y, G23)
        np.testing.assert_allclose(P, st.softmax64(y), rtol=2e-6, atol=1e-9)
    # the float32 grid loses the deep tail: a token 21 nats down is never drawn
    P = _exact_grid_law([0.0, -21.0], G23)
    assert P[1] == 0.0 and st.softmax64([0.0, -21.0])[1] > 7e-10


@pytest.mark.parametrize("fp64", [False, True])
def test_oracle_draws_follow_exact_law(G23, fp64):
    y = np.array([0.4, -0.7, 0.0], dtype=np.float32)
    n = 300_000
    idx = oracle.sample_repeated_row(y, 1.0, seed=5, offset=9, row_ids=np.arange(n), fp64_noise=fp64)
    counts = np.bincount(idx, minlength=3)
    P = _exact_grid_law(y.astype(np.float64), G23)
    assert st.chi2_statistic(counts, P) < st.chi2_quantile(2)


@pytest.mark.parametrize("fp64", [False, True])
def test_chi_square_16_token_row(fp64):
    row = synthetic.chi2_row().numpy()
    n = 1_000_000
    idx = oracle.sample_repeated_row(row, 1.0, seed=1234, offset=0, row_ids=np.arange(n),
                                     fp64_noise=fp64)
    counts = np.bincount(idx, minlength=16)
    chi2 = st.chi2_statistic(counts, st.softmax64(row))
    assert chi2 < st.chi2_quantile(15), chi2


def test_chi_square_fused_with_bias_and_temperature():
    """Law of the fused definition is softmax((y + bias) / T) with y = H W^T."""
    D, V, n, T = 32, 16, 200_000, 0.6
    H1 = synthetic.hidden(1, D, seed=21)
    W = synthetic.weight(V, D, std=0.3, seed=22)
    bias1 = torch.randn((1, V), generator=torch.Generator().manual_seed(23)).float()
    bias1[0, 3] = float("-inf")
    H = H1.expand(n, D).contiguous()
    bias = bias1.expand(n, V).contiguous()
    temp = np.full(n, T, dtype=np.float32)
    idx, _, _ = oracle.sample_fused(H, W, temp, bias.numpy(), seed=77, offset=3,
                                    row_ids=np.arange(n))
    counts = np.bincount(idx, minlength=V)
    y = H1.double().numpy() @ W.double().numpy().T          # independent logits
    p = st.softmax64((y[0] + bias1[0].double().numpy()) / T)
    assert counts[3] == 0 and p[3] == 0.0
    keep = p > 0
    assert st.chi2_statistic(counts[keep], p[keep]) < st.chi2_quantile(int(keep.sum()) - 1)


def _tail_count(V, r, n, fp64, seed=1234, start=0):
    row = synthetic.tail_row(V, r).numpy()
    idx = oracle.sample_repeated_row(row, 1.0, seed=seed, offset=0,
                                     row_ids=np.arange(start, start + n), fp64_noise=fp64)
    return int((idx != 0).sum())


@pytest.mark.parametrize("fp64", [False, True])
def test_tail_rate_moderate_depth(fp64):
    V, r, n = 8193, 6e-6, 16384
    lam = n * st.miss_probability(V, synthetic.tail_depth(r))
    c = _tail_count(V, r, n, fp64)
    assert st.poisson_two_sided_ok(c, lam), (c, lam)


@pytest.mark.slow
def test_tail_rate_page_depth_fp64():
    V, r, n = 131072, 1e-7, 20000
    lam = n * st.miss_probability(V, synthetic.tail_depth(r))
    c = _tail_count(V, r, n, True)
    assert st.poisson_two_sided_ok(c, lam), (c, lam)
