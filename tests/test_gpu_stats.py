"""Sampling-law tests of the GPU path at the Megatron-LM page's sizes ("Tests"):

* tail rate with float64 race noise: rows [0, -D, ..., -D], V = 131072,
  262144 draws per r in {1e-7, 1e-8, 1e-9}; the count of draws that miss token 0
  lies in the two-sided 1e-6 Poisson interval of (V-1) r / (1 + (V-1) r);
* float32-noise non-vacuity: with 23-bit uniforms the count falls below that
  interval at r = 1e-8 and 1e-9 (the representable tail is about 20 nats);
* chi-square over a 16-token row, 1M draws, below the 1e-6 quantile (15 dof);
* on the first 4096 rows of each tail sweep, the draws equal the oracle's.

Every row of a sweep carries the same logits, so one small buffer of logits is
sampled again and again with new logical row ids (the ids key the noise).
"""
import numpy as np
import pytest
import torch

import decode_exact_categorical_amd as fs
import oracle
import synthetic
from gpu_common import check_index_parity, need_gpu, say
from oracle import stats as st

pytestmark = pytest.mark.gpu

V_TAIL = 131072
N_TAIL = 262144
CHUNK = 64           # rows per call: the 32 MB logits buffer stays cache-resident


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _sweep(dev, r, fp64, n=N_TAIL, seed=1234):
    row = synthetic.tail_row(V_TAIL, r)
    x = row.to(dev).expand(CHUNK, V_TAIL).contiguous()
    temp = torch.ones(CHUNK, device=dev)
    out = torch.empty(n, dtype=torch.int64, device=dev)
    ids = torch.arange(n, dtype=torch.int64, device=dev).to(torch.int32)
    for c in range(0, n, CHUNK):
        fs.sample_logits(x, temp, seed=seed, offset=0, row_ids=ids[c:c + CHUNK],
                         fp64_noise=fp64, out=out[c:c + CHUNK])
    torch.cuda.synchronize()
    return out.cpu().numpy(), row.numpy()


@pytest.mark.parametrize("r", [1e-7, 1e-8, 1e-9])
def test_fp64_noise_tail_rate(dev, r):
    say(f"tail rate fp64 r={r}: {N_TAIL} draws of V={V_TAIL}")
    out, row = _sweep(dev, r, True)
    misses = int((out != 0).sum())
    lam = N_TAIL * st.miss_probability(V_TAIL, synthetic.tail_depth(r))
    lo, hi = st.poisson_interval(lam)
    say(f"  misses {misses}, expected {lam:.1f}, accept [{lo}, {hi}]")
    assert st.poisson_two_sided_ok(misses, lam)
    ref, gap = oracle.sample_repeated_row(row, 1.0, seed=1234, offset=0, row_ids=np.arange(4096),
                                          fp64_noise=True, with_gap=True)
    check_index_parity(out[:4096], ref, gap, f"tail r={r} first 4096 rows")


@pytest.mark.parametrize("r", [1e-8, 1e-9])
def test_fp32_noise_misses_tail(dev, r):
    say(f"non-vacuity fp32 r={r}")
    out, _ = _sweep(dev, r, False)
    misses = int((out != 0).sum())
    lam = N_TAIL * st.miss_probability(V_TAIL, synthetic.tail_depth(r))
    lo, hi = st.poisson_interval(lam)
    say(f"  fp32 misses {misses}, softmax interval [{lo}, {hi}]")
    assert misses < lo


@pytest.mark.parametrize("fp64", [False, True])
def test_chi_square_16_token_row(dev, fp64):
    say(f"chi-square 16-token row fp64={fp64}")
    row = synthetic.chi2_row()
    n = 1_000_000
    x = row.to(dev).expand(n, 16).contiguous()
    ids = torch.arange(n, dtype=torch.int32, device=dev)
    out = fs.sample_logits(x, torch.ones(n, device=dev), seed=4321, offset=1, row_ids=ids,
                           fp64_noise=fp64)
    counts = torch.bincount(out, minlength=16).cpu().numpy()
    chi2 = st.chi2_statistic(counts, st.softmax64(row.numpy()))
    say(f"  chi2 = {chi2:.2f} (threshold {st.chi2_quantile(15):.2f})")
    assert chi2 < st.chi2_quantile(15)


def test_chi_square_fused_path(dev):
    """The fused path's law over a 16-token vocabulary with bias and temperature."""
    say("chi-square fused")
    D, V, n, T = 64, 16, 1_000_000, 0.8
    H1 = synthetic.hidden(1, D, seed=41)
    W = synthetic.weight(V, D, std=0.2, seed=42)
    bias1 = torch.randn((1, V), generator=torch.Generator().manual_seed(43))
    Hd = H1.to(dev).expand(n, D).contiguous()
    bd = bias1.to(dev).expand(n, V).contiguous()
    out = fs.sample_fused(Hd, W.to(dev), torch.full((n,), T, device=dev), bd, seed=8, offset=2,
                          row_ids=torch.arange(n, dtype=torch.int32, device=dev))
    counts = torch.bincount(out, minlength=V).cpu().numpy()
    y = oracle.logits(H1, W)[0]
    p = st.softmax64((y + bias1[0].double().numpy()) / T)
    chi2 = st.chi2_statistic(counts, p)
    say(f"  chi2 = {chi2:.2f}")
    assert chi2 < st.chi2_quantile(15)
