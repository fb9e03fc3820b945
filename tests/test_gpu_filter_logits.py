"""GPU parity of fs_filter_logits (the filter chain's output: y / t on the kept
tokens, -inf elsewhere) against the oracle, through the C ABI, and of filtered speculative
decoding composed from it.

* -inf exactly at the oracle's dropped tokens and y / t at its kept tokens
  (within 2.5e-7 relative: the kernel rounds 1/t and then y * (1/t) to
  float32), on every row whose top-p and min-p decisions lie further than
  2e-5 (relative) from their boundaries; per-row settings, V % 4 != 0,
  greedy rows (the largest logit's tie class, unscaled), masks, +inf.
* A draw at temperature 1 from the filtered logits is fs_sample_logits_filtered's
  draw bit for bit (float32 noise, the same per-row kernel).
* Filtered speculative decoding (the spec-decode-ops card: the same filters on
  both models' logits, then verify at temperature 1) against the oracle's
  own composition of filter_logits and verify.
"""
import numpy as np
import pytest
import torch

import decode_exact_categorical_amd as fs
import oracle
import synthetic
from gpu_common import GAP, need_gpu, say

pytestmark = pytest.mark.gpu

FILTER_MARGIN = 2e-5
RTOL = 2.5e-7


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _params(B, setting):
    if setting == "per_row":
        k, p, m = synthetic.filter_settings(B, 100000, seed=41)
        return dict(top_k=k, top_p=p, min_p=m)
    return dict(setting)


def _to_dev(kw, dev):
    return {n: (v.to(dev) if isinstance(v, torch.Tensor) else v) for n, v in kw.items()}


def _to_np(kw):
    return {n: (v.numpy() if isinstance(v, torch.Tensor) else v) for n, v in kw.items()}


CASES = [
    (8, 128256, dict(top_k=50, top_p=0.95)),
    (37, 5003, "per_row"),
    (64, 151936, dict(top_p=0.9)),
    (3, 1000, dict(min_p=0.1)),
    (16, 32768, dict(top_k=1)),
    (5, 777, dict()),
]


@pytest.mark.parametrize("B,V,setting", CASES)
def test_filter_logits_match_oracle(dev, B, V, setting):
    say(f"filter_logits B={B} V={V} {setting}")
    x = synthetic.logits(B, V, seed=40 + B)
    temp = synthetic.temperatures(B, seed=42)
    if B >= 4:
        temp[1] = 0.0                                   # greedy row
        x[2, 5] = float("nan")
        x[2, 7] = -float("inf")
    if B >= 5:
        x[3, 11] = x[3, 12] = float("inf")              # +inf logits keep all the mass
    kw = _params(B, setting)
    got = fs.filter_logits(x.to(dev), temp.to(dev), **_to_dev(kw, dev))
    torch.cuda.synchronize()
    got = got.cpu().double().numpy()
    ref, margin = oracle.filter_logits(x.numpy(), temp.numpy(), **_to_np(kw))
    decided = margin > FILTER_MARGIN
    # top-p over thousands of small masses puts many rows' crossing within the
    # margin: those rows are only checked for structure
    assert decided.mean() >= 0.4
    # every row: kept values are the scaled logits, and the kept set is a value
    # threshold (every kept logit at least every dropped valid one)
    xs = x.numpy().astype(np.float64)
    tt = temp.numpy().astype(np.float64)
    scale = np.where(tt > 0, 1.0 / np.where(tt > 0, tt, 1.0), 1.0)[:, None]
    assert not np.isnan(got).any()
    kept = ~np.isneginf(got)
    np.testing.assert_allclose(got[kept], (xs * scale)[kept], rtol=RTOL)
    valid = ~np.isnan(xs) & ~np.isneginf(xs)
    for b in range(B):
        assert kept[b].any() == valid[b].any()
        dropped = valid[b] & ~kept[b]
        if dropped.any():
            assert xs[b][kept[b]].min() >= xs[b][dropped].max(), f"row {b}"
    for b in np.flatnonzero(decided):
        drop = np.isneginf(ref[b])
        np.testing.assert_array_equal(np.isneginf(got[b]), drop, err_msg=f"row {b}")
        np.testing.assert_allclose(got[b][~drop], ref[b][~drop], rtol=RTOL, err_msg=f"row {b}")


def test_draw_from_filtered_logits_is_the_filtered_draw(dev):
    B, V = 32, 50000                      # B > 24: the per-row kernel on both sides
    say("filtered logits drawn at T = 1 vs the filtered sampler")
    x = synthetic.logits(B, V, seed=43).to(dev)
    temp = synthetic.temperatures(B, seed=44).to(dev)
    for kw in (dict(top_k=50, top_p=0.95), dict(min_p=0.05), dict(top_p=0.5)):
        fl = fs.filter_logits(x, temp, **kw)
        a = fs.sample_logits(fl, torch.ones(B, device=dev), seed=12, offset=34)
        b = fs.sample_logits_filtered(x, temp, seed=12, offset=34, **kw)
        assert torch.equal(a, b), kw


def test_filtered_speculative_decoding(dev):
    B, K, V = 24, 3, 20000
    say("filter_logits on target and draft, then verify at T = 1")
    kw = dict(top_k=100, top_p=0.9)
    target, draft, _ = synthetic.spec_decode(B, K, V, seed=45)
    temp = synthetic.temperatures(B, seed=46)
    t_rows = temp.repeat_interleave(K + 1)
    d_rows = temp.repeat_interleave(K)
    ft_ref, mt = oracle.filter_logits(target.reshape(-1, V).numpy(), t_rows.numpy(), **kw)
    fd_ref, md = oracle.filter_logits(draft.reshape(-1, V).numpy(), d_rows.numpy(), **kw)
    # draft tokens from the filtered draft's own softmax
    g = torch.Generator().manual_seed(47)
    probs = torch.softmax(torch.from_numpy(fd_ref), dim=-1)
    tokens = torch.multinomial(probs, 1, generator=g).reshape(B, K)
    ft = fs.filter_logits(target.reshape(-1, V).to(dev), t_rows.to(dev), **kw)
    fd = fs.filter_logits(draft.reshape(-1, V).to(dev), d_rows.to(dev), **kw)
    acc, out = fs.verify(ft.reshape(B, K + 1, V), fd.reshape(B, K, V), tokens.to(dev),
                         torch.ones(B, device=dev), seed=8, offset=90)
    torch.cuda.synchronize()
    acc, out = acc.cpu().numpy(), out.cpu().numpy()
    r_acc, r_out, margin, gap = oracle.verify(ft_ref.astype(np.float32).reshape(B, K + 1, V),
                                              fd_ref.astype(np.float32).reshape(B, K, V),
                                              tokens.numpy(), np.ones(B, dtype=np.float32),
                                              seed=8, offset=90)
    filt_ok = (mt.reshape(B, K + 1) > FILTER_MARGIN).all(1) & (md.reshape(B, K) > FILTER_MARGIN).all(1)
    decided = filt_ok & (margin > 1e-4)
    assert decided.mean() >= 0.7
    np.testing.assert_array_equal(acc[decided], r_acc[decided])
    rows = np.flatnonzero(decided & (gap > GAP))
    np.testing.assert_array_equal(out[rows, acc[rows]], r_out[rows, r_acc[rows]])
    # every emitted token is inside the target's filtered (kept) set
    for b in range(B):
        L = acc[b]
        assert np.isfinite(ft_ref.reshape(B, K + 1, V)[b, L, out[b, L]])
