"""Pins of the oracle's fused filtered sampling (the logits H W^T summed in
float64, the filter chain temperature -> top-k -> top-p -> min-p over them,
then the draw over the kept tokens), against results pinned elsewhere or
computed independently:

* heads whose logits are exact float32 values (small multiples of 2^-7):
  the fused oracle equals the float32-logits filtered oracle (itself pinned
  against the transformers processors) index for index, gap and margin;
* every filter off: equal to the unfiltered fused oracle draw for draw;
* top_k = 1 and greedy rows: numpy's first argmax of the float64 logits;
* the logit-gap margin at the top-k and top-p cuts on hand-made rows;
* the sampled law of one row drawn under many row ids against the softmax
  over the transformers processors' kept set (chi-square), nothing drawn
  outside it.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import stats


def _exact_head(B, D, V, seed):
    """H[B, D], W[V, D] bf16 holding multiples of 2^-3 and 2^-4 below 2: every
    logit is a multiple of 2^-7 below 2^9 in magnitude, exact in float32."""
    g = torch.Generator().manual_seed(seed)
    H = (torch.randint(-15, 16, (B, D), generator=g).float() / 8).to(torch.bfloat16)
    W = (torch.randint(-15, 16, (V, D), generator=g).float() / 16).to(torch.bfloat16)
    return H, W


SETTINGS = [
    dict(top_k=50),
    dict(top_k=1),
    dict(top_p=0.9),
    dict(top_p=0.3),
    dict(min_p=0.05),
    dict(top_k=40, top_p=0.95),
    dict(top_k=20, top_p=0.5, min_p=0.1),
    dict(top_p=0.8, min_p=0.02),
    dict(top_k=7, top_p=0.0),
    dict(min_p=1.5),
]


@pytest.mark.parametrize("fp64", [False, True])
@pytest.mark.parametrize("setting", SETTINGS)
def test_exact_logits_equal_the_logits_oracle(setting, fp64):
    B, D, V = 24, 64, 3000
    H, W = _exact_head(B, D, V, seed=11)
    y = H.double().numpy() @ W.double().numpy().T
    y32 = y.astype(np.float32)
    assert np.array_equal(y32.astype(np.float64), y)          # exact in float32
    temp = np.linspace(0.4, 1.6, B).astype(np.float32)
    temp[3] = 0.0                                              # a greedy row
    rid = np.arange(B, dtype=np.uint32) * 5 + 2
    a = oracle.sample_fused_filtered(H, W, temp, seed=9, offset=4, row_ids=rid, fp64_noise=fp64,
                                     **setting)
    b = oracle.sample_logits_filtered(y32, temp, seed=9, offset=4, row_ids=rid, fp64_noise=fp64,
                                      **setting)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1], b[1], equal_nan=True)
    assert np.array_equal(a[2], b[2])


@pytest.mark.parametrize("fp64", [False, True])
def test_filters_off_is_the_unfiltered_draw(fp64):
    B, D, V = 16, 256, 5001
    g = torch.Generator().manual_seed(3)
    H = torch.randn(B, D, generator=g).to(torch.bfloat16)
    W = (torch.randn(V, D, generator=g) * 0.05).to(torch.bfloat16)
    temp = np.linspace(0.5, 1.2, B).astype(np.float32)
    temp[0] = float("nan")
    a = oracle.sample_fused_filtered(H, W, temp, top_k=0, top_p=1.0, min_p=0.0, seed=1,
                                     offset=2, fp64_noise=fp64)
    b = oracle.sample_fused(H, W, temp, seed=1, offset=2, fp64_noise=fp64)
    assert np.array_equal(a[0], b[0])
    # the gaps agree on sampled rows; a greedy row keeps only its largest
    # logit's class, so its filtered gap is +inf
    assert np.array_equal(a[1][1:], b[1][1:]) and a[1][0] == np.inf
    assert np.isinf(a[2]).all() and np.isinf(a[3]).all()


def test_top_k_one_and_greedy_are_numpy_argmax():
    B, D, V = 12, 128, 4001
    g = torch.Generator().manual_seed(4)
    H = torch.randn(B, D, generator=g).to(torch.bfloat16)
    W = (torch.randn(V, D, generator=g) * 0.05).to(torch.bfloat16)
    y = H.double().numpy() @ W.double().numpy().T
    ref = np.argmax(y, axis=1)
    temp = np.full(B, 0.8, dtype=np.float32)
    a = oracle.sample_fused_filtered(H, W, temp, top_k=1, seed=5, offset=0)
    assert np.array_equal(a[0], ref)
    a = oracle.sample_fused_filtered(H, W, np.zeros(B, dtype=np.float32), top_p=0.5, min_p=0.1,
                                     seed=5, offset=0)
    assert np.array_equal(a[0], ref)


def test_value_margin_at_the_cuts():
    # H = [1, 0, ...]: the logits are W's first column, chosen by hand
    D = 8
    vals = np.array([3.0, 2.5, 2.25, 1.0, 0.75, -4.0], dtype=np.float32)
    W = torch.zeros((len(vals), D), dtype=torch.bfloat16)
    W[:, 0] = torch.from_numpy(vals).to(torch.bfloat16)
    H = torch.zeros((1, D), dtype=torch.bfloat16)
    H[0, 0] = 1.0
    t = np.ones(1, dtype=np.float32)
    # top-k 2 cuts between 2.5 and 2.25
    _, _, margin, vm = oracle.sample_fused_filtered(H, W, t, top_k=2, seed=0, offset=0)
    assert vm[0] == 0.25 and np.isinf(margin[0])
    # top-p: masses e^0, e^-0.5, e^-0.75, e^-2, e^-2.25, e^-7; p = 0.5 keeps the
    # first two (above 1 < 0.5 Z, then 1 + e^-.5 > 0.5 Z), cutting 2.5 | 2.25
    e = np.exp(vals.astype(np.float64) - 3.0)
    Z = e.sum()
    assert e[0] < 0.5 * Z < e[0] + e[1]
    idx, _, margin, vm = oracle.sample_fused_filtered(H, W, t, top_p=0.5, seed=0, offset=0)
    assert vm[0] == 0.25
    assert np.isclose(margin[0], min(abs(e[0] - 0.5 * Z), abs(e[0] + e[1] - 0.5 * Z)) / Z)
    assert idx[0] in (0, 1)
    # no cut: every filter off leaves both margins infinite
    _, _, margin, vm = oracle.sample_fused_filtered(H, W, t, seed=0, offset=0)
    assert np.isinf(vm[0]) and np.isinf(margin[0])


@pytest.mark.parametrize("setting,fp64", [(dict(top_k=4, top_p=0.8), False),
                                          (dict(min_p=0.1), True),
                                          (dict(top_p=0.6), False)])
def test_sampled_law_against_the_processors(setting, fp64):
    from transformers.generation.logits_process import (MinPLogitsWarper, TemperatureLogitsWarper,
                                                        TopKLogitsWarper, TopPLogitsWarper)
    D, V, T, n = 32, 12, 0.9, 30000
    g = torch.Generator().manual_seed(21)
    H1 = torch.randn(1, D, generator=g).to(torch.bfloat16)
    W = (torch.randn(V, D, generator=g) * 0.4).to(torch.bfloat16)
    y = (H1.double() @ W.double().T)                              # float64 logits [1, V]
    x = TemperatureLogitsWarper(T)(None, y.clone())
    if "top_k" in setting:
        x = TopKLogitsWarper(setting["top_k"])(None, x)
    if "top_p" in setting:
        x = TopPLogitsWarper(setting["top_p"])(None, x)
    if "min_p" in setting:
        x = MinPLogitsWarper(setting["min_p"])(None, x)
    law = torch.softmax(x[0], dim=-1).numpy()
    kept = law > 0
    assert 1 < kept.sum() < V
    H = H1.expand(n, D).contiguous()
    rid = np.arange(n, dtype=np.uint32) * 7 + 3
    idx, _, _, _ = oracle.sample_fused_filtered(H, W, np.full(n, T, dtype=np.float32), seed=8,
                                                offset=1, row_ids=rid, fp64_noise=fp64, **setting)
    assert kept[idx].all()
    counts = np.bincount(idx, minlength=V)[kept]
    chi2 = stats.chi2_statistic(counts, law[kept])
    assert chi2 < stats.chi2_quantile(int(kept.sum()) - 1, 1e-6), chi2
