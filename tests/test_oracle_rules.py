"""Pin the oracle's selection rules.

* Greedy (temperature 0, and by our reading any non-positive or NaN
  temperature): the argmax of y + bias with the smaller index on ties, no noise
  (Triton-sampling skill page, reasoning items 3-4 and correctness
  requirements), checked against numpy's argmax, which returns the first
  occurrence.
* NaN and -inf scores are never selected; a row with none left gives -1;
  masked tokens carry zero mass.
* Seeded draws depend only on (seed, offset, logical row id): they replay,
  survive batch permutation and single-row calls, and change with the offset
  (Megatron-LM "fp64 sampling noise" page, "Tests"; spec-decode-ops page,
  "Determinism").
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic


@pytest.mark.parametrize("t", [0.0, -1.0, float("nan"), -0.0])
def test_greedy_is_first_argmax(t):
    rng = np.random.default_rng(3)
    x = rng.integers(-3, 3, size=(64, 50)).astype(np.float32)   # many exact ties
    idx, gap, _ = oracle.sample_logits(x, np.full(64, t, np.float32), seed=1, offset=2)
    np.testing.assert_array_equal(idx, np.argmax(x, axis=1))
    srt = np.sort(x, axis=1)
    np.testing.assert_array_equal(gap, srt[:, -1] - srt[:, -2])


def test_greedy_fused_uses_bias_before_argmax():
    H = synthetic.hidden(4, 64, seed=5)
    W = synthetic.weight(97, 64, std=0.5, seed=6)
    bias = np.zeros((4, 97), np.float32)
    bias[:, 10] = 1e3
    bias[2, 10] = -np.inf
    idx, _, _ = oracle.sample_fused(H, W, np.zeros(4, np.float32), bias, seed=1, offset=0)
    y = H.double().numpy() @ W.double().numpy().T
    np.testing.assert_array_equal(idx, np.argmax(y + bias, axis=1))
    assert idx[0] == 10 and idx[2] != 10


def test_nan_and_neg_inf_never_selected():
    x = np.full((3, 8), -np.inf, np.float32)
    x[0, 5] = np.nan
    x[1, [2, 6]] = [np.nan, -50.0]
    x[2, [1, 4]] = [np.inf, np.inf]
    for t in (1.0, 0.0):
        idx, gap, _ = oracle.sample_logits(x, np.full(3, t, np.float32), seed=0, offset=0)
        assert idx[0] == -1 and np.isnan(gap[0])
        assert idx[1] == 6 and gap[1] == np.inf
        assert idx[2] == 1                     # +inf ties: smaller index


def test_masked_tokens_have_zero_mass():
    row = synthetic.chi2_row().numpy()
    row[[0, 7, 15]] = -np.inf
    idx = oracle.sample_repeated_row(row, 0.8, seed=2, offset=1, row_ids=np.arange(100_000))
    assert not np.isin(idx, [0, 7, 15]).any()
    assert len(np.unique(idx)) == 13


@pytest.mark.parametrize("fp64", [False, True])
def test_batch_position_invariance_and_replay(fp64):
    B, V = 24, 333
    x = torch.randn((B, V), generator=torch.Generator().manual_seed(8)).numpy()
    temp = np.linspace(0.5, 1.2, B).astype(np.float32)
    rid = np.arange(100, 100 + B, dtype=np.uint32)
    a, _, _ = oracle.sample_logits(x, temp, seed=42, offset=7, row_ids=rid, fp64_noise=fp64)
    a2, _, _ = oracle.sample_logits(x, temp, seed=42, offset=7, row_ids=rid, fp64_noise=fp64)
    np.testing.assert_array_equal(a, a2)
    perm = np.random.default_rng(0).permutation(B)
    p, _, _ = oracle.sample_logits(x[perm], temp[perm], seed=42, offset=7, row_ids=rid[perm],
                                   fp64_noise=fp64)
    np.testing.assert_array_equal(p, a[perm])
    for b in (0, 5, 23):
        s, _, _ = oracle.sample_logits(x[b:b + 1], temp[b:b + 1], seed=42, offset=7,
                                       row_ids=rid[b:b + 1], fp64_noise=fp64)
        assert s[0] == a[b]
    o, _, _ = oracle.sample_logits(x, temp, seed=42, offset=8, row_ids=rid, fp64_noise=fp64)
    assert (o != a).sum() > B // 2


def test_fused_default_row_ids_are_positions():
    H = synthetic.hidden(3, 32, seed=9)
    W = synthetic.weight(50, 32, std=0.5, seed=10)
    t = np.ones(3, np.float32)
    a = oracle.sample_fused(H, W, t, seed=3, offset=4)[0]
    b = oracle.sample_fused(H, W, t, seed=3, offset=4, row_ids=[0, 1, 2])[0]
    np.testing.assert_array_equal(a, b)


def test_infinite_temperature_is_uniform_over_unmasked():
    row = synthetic.chi2_row().numpy()
    row[4] = -np.inf
    n = 150_000
    idx = oracle.sample_repeated_row(row, float("inf"), seed=6, offset=0, row_ids=np.arange(n))
    counts = np.bincount(idx, minlength=16)
    assert counts[4] == 0
    from oracle import stats as st
    keep = np.ones(16, bool)
    keep[4] = False
    assert st.chi2_statistic(counts[keep], np.full(15, 1 / 15)) < st.chi2_quantile(14)
