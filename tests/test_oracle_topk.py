"""Pins of the oracle's Gumbel-top-k (k draws without replacement from the k
largest perturbed scores), independent of the oracle's own selection code:

* the law: the ordered first places follow the Plackett-Luce (sequential
  sampling without replacement) probabilities, written out from softmax, by
  chi-square on rows with 4 tokens, for fp32 and fp64 noise;
* greedy rows: the places equal numpy's stable argsort of the logits;
* masks, NaN and short rows: invalid scores never appear, missing places are
  -1;
* the first place is the single-sample oracle's draw (a different selection
  routine), and the reported scores fall.
"""
import itertools

import numpy as np
import pytest
from scipy import stats

import oracle

P_CHI = 1e-6


def _softmax(y, t):
    z = np.asarray(y, dtype=np.float64) / t
    z = z - z.max()
    p = np.exp(z)
    return p / p.sum()


def _plackett_luce(p, seq):
    prob, left = 1.0, 1.0
    for i in seq:
        prob *= p[i] / left
        left -= p[i]
    return prob


@pytest.mark.parametrize("fp64", [False, True])
@pytest.mark.parametrize("k", [2, 3])
def test_topk_law_is_sampling_without_replacement(k, fp64):
    y = np.array([1.0, 0.5, 0.0, -0.7], dtype=np.float32)
    t = 0.8
    n = 200000
    idx = oracle.topk_repeated_row(y, t, k=k, seed=77, offset=5, row_ids=np.arange(n),
                                   fp64_noise=fp64)
    assert (idx >= 0).all() and (idx < 4).all()
    assert all(len(set(r)) == k for r in idx[:1000].tolist())
    p = _softmax(y, t)
    seqs = list(itertools.permutations(range(4), k))
    expected = np.array([_plackett_luce(p, s) for s in seqs])
    assert abs(expected.sum() - 1.0) < 1e-12
    code = np.zeros(n, dtype=np.int64)
    for j in range(k):
        code = code * 4 + idx[:, j]
    lookup = {sum(v * 4 ** (k - 1 - j) for j, v in enumerate(s)): c for c, s in enumerate(seqs)}
    counts = np.zeros(len(seqs))
    for key, c in zip(*np.unique(code, return_counts=True)):
        counts[lookup[int(key)]] = c
    assert counts.sum() == n
    chi2 = ((counts - n * expected) ** 2 / (n * expected)).sum()
    assert chi2 < stats.chi2.ppf(1 - P_CHI, len(seqs) - 1), chi2


def test_topk_greedy_rows_are_a_stable_sort():
    rng = np.random.default_rng(4)
    x = rng.integers(-3, 3, size=(6, 40)).astype(np.float32)
    temp = np.array([0.0, -1.0, np.nan, 0.0, 0.0, 0.0], dtype=np.float32)
    k = 7
    idx, top = oracle.sample_logits_topk(x, temp, k=k, seed=1, offset=2)
    for b in range(6):
        ref = np.argsort(-x[b].astype(np.float64), kind="stable")[:k]
        np.testing.assert_array_equal(idx[b], ref)
        np.testing.assert_array_equal(top[b, :k], x[b][ref].astype(np.float64))


def test_topk_masks_nan_and_short_rows():
    V, k = 12, 5
    x = np.zeros((4, V), dtype=np.float32)
    x[0, :] = -np.inf
    x[0, [3, 8]] = [1.0, 2.0]                  # two valid entries
    x[1, :] = np.nan
    x[1, 5] = 0.0                              # one valid entry
    x[2, ::2] = -np.inf                        # odd indices only
    x[3, :] = -np.inf                          # none
    idx, top = oracle.sample_logits_topk(x, np.ones(4, np.float32), k=k, seed=3, offset=4)
    assert sorted(idx[0, :2].tolist()) == [3, 8] and (idx[0, 2:] == -1).all()
    assert idx[1, 0] == 5 and (idx[1, 1:] == -1).all()
    assert (idx[2] % 2 == 1).all() and len(set(idx[2].tolist())) == k
    assert (idx[3] == -1).all() and np.isneginf(top[3]).all()
    assert np.isneginf(top[0, 2:]).all() and np.isneginf(top[1, 1:]).all()


@pytest.mark.parametrize("fp64", [False, True])
def test_topk_first_place_is_the_single_draw(fp64):
    rng = np.random.default_rng(5)
    B, V, k = 16, 3000, 6
    x = (rng.standard_normal((B, V)) * 2).astype(np.float32)
    temp = rng.uniform(0.5, 1.5, B).astype(np.float32)
    temp[3] = 0.0
    rid = np.arange(100, 100 + B, dtype=np.uint32)
    idx, top = oracle.sample_logits_topk(x, temp, k=k, seed=9, offset=10, row_ids=rid,
                                         fp64_noise=fp64)
    one, _, best = oracle.sample_logits(x, temp, seed=9, offset=10, row_ids=rid, fp64_noise=fp64)
    np.testing.assert_array_equal(idx[:, 0], one)
    np.testing.assert_array_equal(top[:, 0], best)
    assert (np.diff(top, axis=1) <= 0).all()
    assert all(len(set(r)) == k for r in idx.tolist())
