"""GPU parity of filtered exact sampling fused into the LM head
(fs_sample_fused_filtered), through the C ABI.

* Against the materialised path on the same float32 logits: the fused call
  draws what fs_sample_logits_filtered draws over fs_debug_logits(H, W) (the
  same matmul code, 64-row slices so that both use tiles of at most 64
  columns), bit for bit on every row with top-k on, with top-p off, or whose
  top-p decisions lie further than 1e-5 (relative) from their boundaries
  (rows with top-p but no top-k total their mass from the tiles' float64 sums;
  either side's margin rule is that of the filtered sampler).
* Against the oracle (float64 logits, its own filter chain and draw): the
  GPU logits within 2e-3 of the oracle's; the index equal on every row whose
  top-p / min-p decisions lie further than 1e-4 from their boundaries, whose
  top-k / top-p cuts separate logits further apart than twice the measured
  largest logit error of the case (no reordering across a cut), and whose
  kept top-2 perturbed-score gap exceeds 1e-3; a floor on the number of
  compared rows.
* Rows the tiles' lists cannot resolve (top-p alone over flat rows, min-p over
  flat rows) go through the exact fallback inside the call and still match.
* Per-row mixes of the filters, greedy rows, fp32 and fp64 noise, ragged V,
  several batch tiles; replay and batch permutation with row ids; the
  workspace's counters and flags are left at zero.
* Full size: the Qwen3-8B-shaped head (D = 4096, V = 151936) with the card's
  settings (top_k 50, top_p 0.95) at B = 1, 8, 64, every row against the
  oracle and the materialised path.
"""
import numpy as np
import pytest
import torch

import decode_exact_categorical_amd as fs
import oracle
import synthetic
from gpu_common import GAP, LOGIT_TOL, need_gpu, say

pytestmark = pytest.mark.gpu

MASS_MARGIN = 1e-4          # oracle mass-decision margin (relative)
MAT_MARGIN = 1e-5           # top-p rows without top-k compared with the materialised path


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _head(B, D, V, std, seed):
    H = synthetic.hidden(B, D, seed=seed)
    W = synthetic.weight(V, D, std=std, seed=seed + 1)
    return H, W


def _params(B, V, seed, greedy_rows=(2,)):
    k, p, m = synthetic.filter_settings(B, V, seed=seed)
    t = synthetic.temperatures(B, seed=seed + 1)
    for r in greedy_rows:
        if r < B:
            t[r] = 0.0
    return t, k, p, m


def _fused(dev, H, Wd, t, k, p, m, *, seed, offset, fp64, row_ids=None):
    got = fs.sample_fused_filtered(H.to(dev), Wd, t.to(dev), top_k=k.to(dev), top_p=p.to(dev),
                                   min_p=m.to(dev), seed=seed, offset=offset,
                                   row_ids=None if row_ids is None else row_ids.to(dev),
                                   fp64_noise=fp64)
    torch.cuda.synchronize()
    return got.cpu().numpy()


def _materialised(dev, H, Wd, t, k, p, m, *, seed, offset, fp64, row_ids=None):
    """fs_sample_logits_filtered over fs_debug_logits, 64 rows at a time."""
    out = []
    for r0 in range(0, H.shape[0], 64):
        sl = slice(r0, r0 + 64)
        Y = fs.debug_logits(H[sl].to(dev), Wd)
        rid = (torch.arange(r0, min(H.shape[0], r0 + 64), dtype=torch.int32) if row_ids is None
               else row_ids[sl])
        o = fs.sample_logits_filtered(Y, t[sl].to(dev), top_k=k[sl].to(dev), top_p=p[sl].to(dev),
                                      min_p=m[sl].to(dev), seed=seed, offset=offset,
                                      row_ids=rid.to(dev), fp64_noise=fp64)
        out.append(o.cpu().numpy())
    torch.cuda.synchronize()
    return np.concatenate(out)


def _logit_error(dev, H, W, Wd, rows):
    """Largest |GPU logit - float64 logit| over the given rows (fs_debug_logits
    against the oracle's sums), checked against the logit tolerance."""
    err = 0.0
    for r in rows:
        y = fs.debug_logits(H[r:r + 1].to(dev), Wd)[0].cpu().double().numpy()
        err = max(err, float(np.abs(y - oracle.logits(H[r:r + 1], W)[0]).max()))
    assert err <= LOGIT_TOL, err
    return err


def _check_oracle(got, ref, what, err, min_frac=0.5):
    idx, gap, margin, vmargin = ref
    ok = (margin > MASS_MARGIN) & (vmargin > 2 * err) & ((gap > GAP) | (idx == -1))
    bad = np.flatnonzero(ok & (got != idx))
    assert bad.size == 0, (f"{what}: rows {bad[:5]} got {got[bad[:5]]} oracle {idx[bad[:5]]} "
                           f"gap {gap[bad[:5]]} margin {margin[bad[:5]]} vmargin {vmargin[bad[:5]]}")
    assert ok.mean() >= min_frac, (what, ok.mean())
    say(f"  {what}: {int(ok.sum())} of {len(got)} rows compared with the oracle, all equal "
        f"(logit error {err:.2e})")


def _check_materialised(got, mat, k, p, ref, what):
    k, p = k.numpy(), p.numpy()
    topp_only = (p < 1.0) & (p > 0.0) & ~(k > 0)
    strict = ~topp_only | (ref[2] > MAT_MARGIN)
    bad = np.flatnonzero(strict & (got != mat))
    assert bad.size == 0, f"{what}: rows {bad[:5]} fused {got[bad[:5]]} materialised {mat[bad[:5]]}"
    say(f"  {what}: {int(strict.sum())} of {len(got)} rows equal to the materialised path "
        f"({int((~strict & (got != mat)).sum())} near-boundary rows differ)")


CASES = [
    dict(B=1, D=256, V=3001, std=0.05),
    dict(B=5, D=512, V=20000, std=0.05),
    dict(B=37, D=256, V=50001, std=0.08),
    dict(B=64, D=512, V=32768, std=0.05),
    dict(B=100, D=256, V=9001, std=0.05),       # two batch tiles
    dict(B=24, D=256, V=40000, std=0.005),      # flat rows: the fallback path
]


@pytest.mark.parametrize("fp64", [False, True])
@pytest.mark.parametrize("case", CASES)
def test_fused_filtered_parity(dev, case, fp64):
    B, D, V, std = case["B"], case["D"], case["V"], case["std"]
    say(f"fused filtered B={B} D={D} V={V} std={std} fp64={fp64}")
    H, W = _head(B, D, V, std, seed=500 + B)
    t, k, p, m = _params(B, V, seed=510 + B)
    rid = torch.arange(B, dtype=torch.int32) * 3 + 7
    Wd = W.to(dev)
    got = _fused(dev, H, Wd, t, k, p, m, seed=77, offset=9, fp64=fp64, row_ids=rid)
    mat = _materialised(dev, H, Wd, t, k, p, m, seed=77, offset=9, fp64=fp64, row_ids=rid)
    say("  oracle")
    ref = oracle.sample_fused_filtered(H, W, t.numpy(), top_k=k.numpy(), top_p=p.numpy(),
                                       min_p=m.numpy(), seed=77, offset=9,
                                       row_ids=rid.numpy().astype(np.uint32), fp64_noise=fp64)
    _check_materialised(got, mat, k, p, ref, f"B={B} V={V}")
    err = _logit_error(dev, H, W, Wd, range(min(B, 4)))
    _check_oracle(got, ref, f"B={B} V={V}", err, min_frac=0.25 if B >= 24 else 0.0)


def test_fallback_rows_and_workspace(dev):
    """Top-p alone over flat rows keeps far more tokens than the tiles' lists
    hold: those rows take the fallback inside the call, which is the filtered
    sampler's one-workgroup path over the same logits, so every row equals
    fs_sample_logits_filtered on fs_debug_logits bit for bit (at V <= 8192 that
    call runs the same one-workgroup path); the workspace's counter region is
    left at zero."""
    B, D, V = 16, 256, 6000
    say("fused filtered fallback rows")
    H, W = _head(B, D, V, 0.004, seed=600)
    t = torch.full((B,), 1.0)
    k = torch.zeros(B, dtype=torch.int32)
    p = torch.where(torch.arange(B) % 2 == 0, torch.tensor(0.9), torch.tensor(1.0)).float()
    m = torch.where(torch.arange(B) % 2 == 1, torch.tensor(0.2), torch.tensor(0.0)).float()
    Wd = W.to(dev)
    got = _fused(dev, H, Wd, t, k, p, m, seed=5, offset=1, fp64=False)
    mat = _materialised(dev, H, Wd, t, k, p, m, seed=5, offset=1, fp64=False)
    ref = oracle.sample_fused_filtered(H, W, t.numpy(), top_k=k.numpy(), top_p=p.numpy(),
                                       min_p=m.numpy(), seed=5, offset=1)
    kept, _ = oracle.filter_kept(fs.debug_logits(H.to(dev), Wd).cpu().numpy(), t.numpy(),
                                 top_k=k.numpy(), top_p=p.numpy(), min_p=m.numpy())
    # the top-p rows keep far more than the 8 logits each tile lists
    assert (kept[::2].sum(axis=1) > 8 * fs.fused_tiles(B, D, V)).all()
    assert np.array_equal(got, mat), (got, mat)
    err = _logit_error(dev, H, W, Wd, range(2))
    _check_oracle(got, ref, "fallback rows", err, min_frac=0.25)
    ws = fs._workspace(dev, 0)
    assert int(ws[: 4 * (B + 1)].view(torch.int32).abs().sum().item()) == 0


def test_replay_and_permutation(dev):
    B, D, V = 48, 256, 30011
    say("fused filtered replay and permutation")
    H, W = _head(B, D, V, 0.05, seed=700)
    t, k, p, m = _params(B, V, seed=710)
    rid = torch.arange(B, dtype=torch.int32) + 1000
    Wd = W.to(dev)
    a = _fused(dev, H, Wd, t, k, p, m, seed=3, offset=4, fp64=False, row_ids=rid)
    b = _fused(dev, H, Wd, t, k, p, m, seed=3, offset=4, fp64=False, row_ids=rid)
    assert np.array_equal(a, b)
    perm = torch.randperm(B, generator=torch.Generator().manual_seed(7))
    c = _fused(dev, H[perm], Wd, t[perm], k[perm], p[perm], m[perm], seed=3, offset=4,
               fp64=False, row_ids=rid[perm])
    assert np.array_equal(c, a[perm.numpy()])


@pytest.fixture(scope="module")
def qwen_head(dev):
    say("generating the D=4096 V=151936 head")
    W = synthetic.weight(151936, 4096, std=0.02)
    H = synthetic.hidden(64, 4096)
    temp = synthetic.temperatures(64)
    return H, W, temp, W.to(dev)


@pytest.mark.parametrize("B", [1, 8, 64])
def test_qwen_head_card_settings(dev, qwen_head, B):
    H, W, temp, Wd = qwen_head
    say(f"fused filtered Qwen head B={B}: top_k 50, top_p 0.95")
    k = torch.full((B,), 50, dtype=torch.int32)
    p = torch.full((B,), 0.95)
    m = torch.zeros(B)
    got = _fused(dev, H[:B], Wd, temp[:B], k, p, m, seed=1234, offset=17, fp64=False)
    mat = _materialised(dev, H[:B], Wd, temp[:B], k, p, m, seed=1234, offset=17, fp64=False)
    assert np.array_equal(got, mat)
    ref = oracle.sample_fused_filtered(H[:B], W, temp[:B].numpy(), top_k=50, top_p=0.95,
                                       seed=1234, offset=17)
    err = _logit_error(dev, H, W, Wd, (0, B - 1))
    _check_oracle(got, ref, f"qwen B={B}", err, min_frac=0.5)
