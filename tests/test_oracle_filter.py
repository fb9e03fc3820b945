"""Pins of the oracle's filtered sampling (temperature -> top-k -> top-p ->
min-p -> Gumbel draw over the kept tokens), independent of the oracle's own
code:

* kept sets against the transformers library's own logits processors
  (TemperatureLogitsWarper, TopKLogitsWarper, TopPLogitsWarper,
  MinPLogitsWarper, applied in that order), on rows without ties and on rows
  full of ties (where the processors' top-p keeps a sort-order-dependent part
  of the boundary tie class and the oracle keeps all of it);
* hand-worked rows with known probabilities (the crossing token of top-p);
* the sampled law on a small row against the softmax over the processors'
  kept set (chi-square), with no draw outside it;
* special cases that reduce to other pinned results: every filter off equals
  the unfiltered sampler draw for draw, top_k = 1 is numpy's argmax, greedy
  rows, masks and NaN;
* the filtered logits (filter_logits) against the processors' own output
  values: -inf at the same tokens, y / t elsewhere;
* the repetition penalty against the transformers processor
  (RepetitionPenaltyLogitsProcessor) bit for bit, duplicates and padding
  included.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import stats

MARGIN = 1e-4     # rows whose top-p / min-p decision is closer than this are set aside


def _processors_kept(row, t, top_k, top_p, min_p):
    """Kept mask of one row under the transformers processors."""
    from transformers.generation.logits_process import (MinPLogitsWarper, TemperatureLogitsWarper,
                                                        TopKLogitsWarper, TopPLogitsWarper)
    x = torch.as_tensor(np.asarray(row, dtype=np.float32))[None].clone()
    x = TemperatureLogitsWarper(float(t))(None, x)
    if top_k is not None:
        x = TopKLogitsWarper(int(top_k))(None, x)
    if top_p is not None:
        x = TopPLogitsWarper(float(top_p))(None, x)
    if min_p is not None:
        x = MinPLogitsWarper(float(min_p))(None, x)
    return (x[0] != -float("inf")).numpy()


SETTINGS = [
    dict(top_k=50),
    dict(top_k=1),
    dict(top_p=0.9),
    dict(top_p=0.3),
    dict(min_p=0.05),
    dict(min_p=0.5),
    dict(top_k=40, top_p=0.95),
    dict(top_k=20, top_p=0.5, min_p=0.1),
    dict(top_p=0.8, min_p=0.02),
    dict(top_k=200, min_p=0.2),
]


@pytest.mark.parametrize("setting", SETTINGS)
def test_kept_set_matches_transformers_processors(setting):
    rng = np.random.default_rng(11)
    B, V = 60, 300
    x = (rng.standard_normal((B, V)) * rng.uniform(0.5, 4.0, size=(B, 1))).astype(np.float32)
    t = rng.uniform(0.3, 1.5, size=B).astype(np.float32)
    kept, margin = oracle.filter_kept(x, t, **setting)
    checked = 0
    for b in range(B):
        if margin[b] <= MARGIN:
            continue
        ref = _processors_kept(x[b], t[b], setting.get("top_k"), setting.get("top_p"),
                               setting.get("min_p"))
        np.testing.assert_array_equal(kept[b], ref, err_msg=f"row {b} {setting}")
        checked += 1
    assert checked >= 0.8 * B


@pytest.mark.parametrize("setting", [dict(top_k=7), dict(top_k=3, min_p=0.3), dict(top_p=0.6),
                                     dict(top_k=10, top_p=0.7)])
def test_kept_set_with_ties(setting):
    """Logits on a coarse grid (many ties).  Top-k keeps a tie at the k-th value
    whole, as the processors do.  Top-p: the oracle keeps the boundary tie class
    whole; the processors keep a part of it that depends on their sort order."""
    rng = np.random.default_rng(12)
    B, V = 80, 64
    x = np.round(rng.standard_normal((B, V)) * 2) / 2
    x = x.astype(np.float32)
    t = np.full(B, 0.9, dtype=np.float32)
    kept, margin = oracle.filter_kept(x, t, **setting)
    for b in range(B):
        if margin[b] <= MARGIN:
            continue
        ref = _processors_kept(x[b], t[b], setting.get("top_k"), setting.get("top_p"),
                               setting.get("min_p"))
        if "top_p" not in setting:
            np.testing.assert_array_equal(kept[b], ref, err_msg=f"row {b}")
            continue
        assert (ref <= kept[b]).all(), f"row {b}: a processor-kept token dropped"
        extra = np.unique(x[b][kept[b] & ~ref])
        assert extra.size <= 1, f"row {b}: extra tokens span {extra}"
        if extra.size:
            assert ref[x[b] == extra[0]].any(), "the extra tokens complete a kept tie class"


def test_top_p_crossing_token_and_min_p_by_hand():
    # probabilities 0.5, 0.3, 0.2 (temperature 1)
    x = np.log(np.array([[0.5, 0.3, 0.2]], dtype=np.float64)).astype(np.float32)
    t = [1.0]
    for p, want in ((0.4, [1, 0, 0]), (0.6, [1, 1, 0]), (0.85, [1, 1, 1]), (0.95, [1, 1, 1])):
        np.testing.assert_array_equal(oracle.filter_kept(x, t, top_p=p)[0][0], np.array(want) > 0)
    # min-p keeps p >= m * 0.5
    for m, want in ((0.3, [1, 1, 1]), (0.5, [1, 1, 0]), (0.7, [1, 0, 0]), (2.0, [1, 0, 0])):
        np.testing.assert_array_equal(oracle.filter_kept(x, t, min_p=m)[0][0], np.array(want) > 0)
    # margins: the distance of the closest decision from its boundary; the
    # largest token's class decides nothing (mass above 0, mass ratio 1)
    for kw, want in ((dict(top_p=0.6), 0.1), (dict(top_p=0.85), 0.05), (dict(top_p=0.05), 0.45),
                     (dict(min_p=0.5), 0.2),
                     (dict(min_p=1.0), 0.4), (dict(top_p=0.0), np.inf), (dict(top_k=2), np.inf)):
        got = oracle.filter_kept(x, t, **kw)[1][0]
        assert (got == want) if np.isinf(want) else abs(got - want) < 1e-6, (kw, got)
    # top-p after top-k renormalises over the top-k survivors: 0.5 / 0.8 = 0.625
    np.testing.assert_array_equal(oracle.filter_kept(x, t, top_k=2, top_p=0.6)[0][0], [1, 0, 0])
    np.testing.assert_array_equal(oracle.filter_kept(x, t, top_k=2, top_p=0.65)[0][0], [1, 1, 0])


def test_filters_off_and_degenerate_values():
    rng = np.random.default_rng(13)
    B, V = 6, 50
    x = rng.standard_normal((B, V)).astype(np.float32)
    x[1, 3] = -np.inf
    x[2, 7] = np.nan
    t = np.full(B, 0.8, dtype=np.float32)
    valid = ~np.isnan(x) & (x != -np.inf)
    for kw in (dict(top_k=0), dict(top_k=V), dict(top_k=-5), dict(top_p=1.0), dict(top_p=np.nan),
               dict(min_p=0.0), dict(min_p=np.nan), dict()):
        kept, margin = oracle.filter_kept(x, t, **kw)
        np.testing.assert_array_equal(kept, valid, err_msg=str(kw))
    # a filter that would keep nothing keeps the largest logit's tie class
    y = x.copy()
    y[0, 10] = y[0, 20] = 9.0
    for kw in (dict(top_p=0.0), dict(top_p=-1.0), dict(min_p=1.5)):
        kept, _ = oracle.filter_kept(y, t, **kw)
        assert set(np.flatnonzero(kept[0])) == {10, 20}, kw


def test_no_filter_equals_unfiltered_sampler():
    rng = np.random.default_rng(14)
    B, V = 24, 700
    x = (rng.standard_normal((B, V)) * 2).astype(np.float32)
    x[3, :] = -np.inf                       # fully masked
    x[4, ::3] = np.nan
    x[5, 100] = np.inf
    t = rng.uniform(0.5, 1.2, size=B).astype(np.float32)
    t[6], t[7], t[8] = 0.0, -1.0, np.nan     # greedy
    for fp64 in (False, True):
        a, _, _ = oracle.sample_logits(x, t, seed=5, offset=9, fp64_noise=fp64)
        b, _, margin = oracle.sample_logits_filtered(x, t, seed=5, offset=9, fp64_noise=fp64)
        np.testing.assert_array_equal(a, b)
        assert np.isinf(margin).all()
    # top_k = V keeps everything too
    a, _, _ = oracle.sample_logits(x, t, seed=5, offset=9)
    b, _, _ = oracle.sample_logits_filtered(x, t, top_k=V, seed=5, offset=9)
    np.testing.assert_array_equal(a, b)


def test_top_k_one_is_argmax_and_greedy_rows():
    rng = np.random.default_rng(15)
    B, V = 40, 500
    x = rng.standard_normal((B, V)).astype(np.float32)
    t = rng.uniform(0.5, 1.5, size=B).astype(np.float32)
    idx, _, _ = oracle.sample_logits_filtered(x, t, top_k=1, seed=1, offset=2)
    np.testing.assert_array_equal(idx, np.argmax(x, axis=1))
    t0 = np.zeros(B, dtype=np.float32)
    idx, _, _ = oracle.sample_logits_filtered(x, t0, top_k=30, top_p=0.5, min_p=0.3, seed=1, offset=2)
    np.testing.assert_array_equal(idx, np.argmax(x, axis=1))
    # a greedy row keeps the largest logit's tie class, whatever the filters
    x[3, 17] = x[3, 230] = x[3].max() + 1
    kept, _ = oracle.filter_kept(x, t0, top_k=30, top_p=0.99)
    np.testing.assert_array_equal(kept, x == x.max(axis=1, keepdims=True))


def test_masks_never_kept_and_all_masked_row():
    x = np.array([[-np.inf, np.nan, 1.0, 0.5],
                  [-np.inf, -np.inf, np.nan, -np.inf],
                  [0.0, np.inf, 3.0, np.inf]], dtype=np.float32)
    t = np.ones(3, dtype=np.float32)
    kept, _ = oracle.filter_kept(x, t, top_p=0.99)
    assert not kept[0, 0] and not kept[0, 1] and not kept[1].any()
    np.testing.assert_array_equal(kept[2], [False, True, False, True])   # +inf holds all the mass
    idx, _, _ = oracle.sample_logits_filtered(x, t, top_k=3, min_p=0.1, seed=3, offset=4)
    assert idx[1] == -1
    assert idx[2] == 1                   # +inf ties: the smaller index


@pytest.mark.parametrize("fp64", [False, True])
def test_law_chi_square(fp64):
    row = np.array([2.0, 1.6, 1.5, 1.0, 0.9, 0.2, -0.3, -1.0, 0.7, 1.55], dtype=np.float32)
    t, k, p, m = 0.8, 7, 0.85, 0.08
    ref_kept = _processors_kept(row, t, k, p, m)
    z = row.astype(np.float64) / t
    law = np.where(ref_kept, np.exp(z - z.max()), 0.0)
    law /= law.sum()
    n = 200000
    rid = np.arange(n, dtype=np.uint32)
    draws = oracle.filtered_repeated_row(row, t, top_k=k, top_p=p, min_p=m, seed=77, offset=3,
                                         row_ids=rid, fp64_noise=fp64)
    counts = np.bincount(draws, minlength=row.size)
    assert counts[~ref_kept].sum() == 0
    keep = np.flatnonzero(ref_kept)
    chi2 = stats.chi2_statistic(counts[keep], law[keep])
    thr = stats.chi2_quantile(keep.size - 1, 1e-6)
    assert chi2 < thr, (chi2, thr)


@pytest.mark.parametrize("setting", SETTINGS[:6] + [dict()])
def test_filter_logits_match_processor_output(setting):
    """The processors' own output: y / t on the tokens they keep, -inf elsewhere."""
    rng = np.random.default_rng(16)
    B, V = 40, 300
    x = (rng.standard_normal((B, V)) * rng.uniform(0.5, 4.0, size=(B, 1))).astype(np.float32)
    t = rng.uniform(0.3, 1.5, size=B).astype(np.float32)
    out, margin = oracle.filter_logits(x, t, **setting)
    from transformers.generation.logits_process import (MinPLogitsWarper, TemperatureLogitsWarper,
                                                        TopKLogitsWarper, TopPLogitsWarper)
    checked = 0
    for b in range(B):
        if margin[b] <= MARGIN:
            continue
        z = TemperatureLogitsWarper(float(t[b]))(None, torch.as_tensor(x[b])[None].clone())
        if "top_k" in setting:
            z = TopKLogitsWarper(setting["top_k"])(None, z)
        if "top_p" in setting:
            z = TopPLogitsWarper(setting["top_p"])(None, z)
        if "min_p" in setting:
            z = MinPLogitsWarper(setting["min_p"])(None, z)
        z = z[0].double().numpy()
        np.testing.assert_array_equal(np.isinf(out[b]) & (out[b] < 0), np.isinf(z) & (z < 0))
        fin = np.isfinite(z)
        np.testing.assert_allclose(out[b][fin], z[fin], rtol=2e-7)
        checked += 1
    assert checked >= 0.8 * B


def test_filter_logits_greedy_and_masks():
    x = np.array([[1.0, 3.0, np.nan, 3.0, -np.inf], [0.5, -1.0, 2.0, 1.0, 0.0]], dtype=np.float32)
    out, _ = oracle.filter_logits(x, [0.0, 2.0], top_k=2)
    np.testing.assert_array_equal(out[0], [-np.inf, 3.0, -np.inf, 3.0, -np.inf])
    np.testing.assert_array_equal(out[1], [-np.inf, -np.inf, 1.0, 0.5, -np.inf])


def test_repetition_penalty_matches_transformers():
    from transformers.generation.logits_process import RepetitionPenaltyLogitsProcessor
    rng = np.random.default_rng(17)
    B, V, L = 12, 500, 40
    x = (rng.standard_normal((B, V)) * 3).astype(np.float32)
    x[0, :5] = 0.0
    x[1, 7] = -np.inf
    prev = rng.integers(0, V, (B, L))
    prev[:, 1] = prev[:, 0]                       # duplicates count once
    prev[0, :5] = np.arange(5)                    # zero logits: 0 / p
    prev[1, 0] = 7
    for pen in (1.3, 0.7, 2.0):
        ref = RepetitionPenaltyLogitsProcessor(pen)(torch.from_numpy(prev),
                                                    torch.from_numpy(x.copy())).numpy()
        got = oracle.repetition_penalty(x, prev, pen)
        np.testing.assert_array_equal(got, ref)
    # padding outside [0, V) is ignored; a penalty that is not positive is off
    pp = prev.copy()
    pp[:, L // 2:] = -1
    pp[:, -1] = V
    ref = RepetitionPenaltyLogitsProcessor(1.5)(torch.from_numpy(prev[:, :L // 2]),
                                                torch.from_numpy(x.copy())).numpy()
    np.testing.assert_array_equal(oracle.repetition_penalty(x, pp, 1.5), ref)
    np.testing.assert_array_equal(oracle.repetition_penalty(x, prev, 0.0), x)
