"""GPU parity of filtered exact sampling (fs_sample_logits_filtered) against
the oracle, through the C ABI.

* Index parity: every row whose filter decisions are further than 2e-5 from
  their boundaries (the oracle's margin, relative) and whose top-2 kept
  perturbed-score gap exceeds 1e-3 draws the oracle's token; per-row mixes of
  top-k, top-p and min-p, float32 and float64 noise, ragged V, greedy, masked
  and NaN rows.
* Every draw lies in the oracle's kept set, over many offsets.
* A row with every filter off draws exactly what fs_sample_logits draws.
* Every launch shape: one workgroup per row (large batches, short rows) and
  rows split over several workgroups whose candidate lists are merged per
  row, in the row's last workgroup (B <= 8) or in a second launch (9 to 96
  rows), including rows whose lists cannot hold the kept set (the merge then
  runs the one-workgroup path).
* The law of the draws on a small row (chi-square against the softmax over the
  kept set) and zero draws outside it.
* Full size: the Qwen3-8B-shaped vocabulary (V = 151936), B = 8 (split rows,
  one launch) and B = 64 (split rows, two launches), every row against the
  oracle.
"""
import numpy as np
import pytest
import torch

import decode_exact_categorical_amd as fs
import oracle
import synthetic
from gpu_common import check_index_parity, need_gpu, say
from oracle import stats

pytestmark = pytest.mark.gpu
# The kernel's masses are float32 exp((y - M) * (1/t)): three float32 roundings
# in the exponent x (relative error <= 3 * 2^-24 * |x|, at most 7e-6 for the
# |x| <= 40 that carry mass above the 2^-40 fixed-point unit) and one ulp of
# exp; the fixed-point sums lose at most V * 2^-40 of the largest token's mass.
# A top-p or min-p decision further than 2e-5 (relative) from its boundary is
# therefore taken the same way on both sides.
MARGIN = 2e-5


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _run(dev, x, t, k, p, m, *, seed, offset, fp64=False, row_ids=None):
    dx = x.to(dev)
    dt = t.to(dev)
    dk = None if k is None else k.to(dev)
    dp = None if p is None else p.to(dev)
    dm = None if m is None else m.to(dev)
    drid = None if row_ids is None else row_ids.to(dev)
    got = fs.sample_logits_filtered(dx, dt, top_k=dk, top_p=dp, min_p=dm, seed=seed, offset=offset,
                                    row_ids=drid, fp64_noise=fp64)
    torch.cuda.synchronize()
    return got.cpu().numpy()


def _oracle(x, t, k, p, m, *, seed, offset, fp64=False, row_ids=None):
    npf = lambda v: None if v is None else v.numpy()
    return oracle.sample_logits_filtered(x.numpy(), t.numpy(), top_k=npf(k), top_p=npf(p),
                                         min_p=npf(m), seed=seed, offset=offset,
                                         row_ids=None if row_ids is None else row_ids.numpy(),
                                         fp64_noise=fp64)


def _check(got, idx, gap, margin, what):
    # rows whose kept set rounding may decide are compared like near ties
    gap = np.where(margin > MARGIN, gap, 0.0)
    near = check_index_parity(got, idx, gap, what)
    assert near <= max(2, got.size // 4), f"{what}: {near} undecided rows"


CASES = [
    dict(B=37, V=1001),
    dict(B=16, V=5003),              # V % 4 != 0: scalar loads
    dict(B=8, V=32768),
    dict(B=64, V=2048, std=1.0),     # flatter rows: large top-p sets
    dict(B=5, V=7),
    dict(B=3, V=1),
    dict(B=600, V=9000),             # one workgroup per row
    dict(B=8, V=20000),              # the most rows split in one launch
    dict(B=24, V=20000),             # split rows, chunks and merges in two launches
    dict(B=96, V=20000),             # the most rows split in two launches
    dict(B=97, V=20000),             # one workgroup per row again
    dict(B=4, V=262144),             # the most chunks a split row has
    dict(B=40, V=262144),            # ... in two launches
]


@pytest.mark.parametrize("fp64", [False, True])
@pytest.mark.parametrize("case", CASES)
def test_filtered_parity_mixed_settings(dev, case, fp64):
    B, V = case["B"], case["V"]
    say(f"filtered parity B={B} V={V} fp64={fp64}")
    x = synthetic.logits(B, V, std=case.get("std", 3.0), seed=50 + V)
    t = synthetic.temperatures(B, seed=51)
    k, p, m = synthetic.filter_settings(B, V, seed=52 + B)
    got = _run(dev, x, t, k, p, m, seed=99, offset=7, fp64=fp64)
    idx, gap, margin = _oracle(x, t, k, p, m, seed=99, offset=7, fp64=fp64)
    _check(got, idx, gap, margin, f"B={B} V={V} fp64={fp64}")


@pytest.mark.parametrize("setting", [dict(top_k=1), dict(top_k=50), dict(top_p=0.9),
                                     dict(min_p=0.05), dict(top_k=40, top_p=0.95, min_p=0.02),
                                     dict(top_p=0.0), dict(min_p=1.0), dict(min_p=3.0),
                                     dict(top_k=2000, top_p=0.3), dict(top_k=3000, min_p=0.3),
                                     dict(top_k=9000), dict(top_k=9000, top_p=0.6)])
def test_filtered_parity_uniform_settings(dev, setting):
    B, V = 48, 12345
    say(f"filtered parity {setting}")
    x = synthetic.logits(B, V, seed=60)
    t = synthetic.temperatures(B, seed=61)
    conv = {"top_k": torch.int32, "top_p": torch.float32, "min_p": torch.float32}
    full = {n: (torch.full((B,), v, dtype=conv[n]) if n in setting else None)
            for n, v in [("top_k", setting.get("top_k", 0)), ("top_p", setting.get("top_p", 1.0)),
                         ("min_p", setting.get("min_p", 0.0))]}
    got = _run(dev, x, t, full["top_k"], full["top_p"], full["min_p"], seed=3, offset=4)
    idx, gap, margin = _oracle(x, t, full["top_k"], full["top_p"], full["min_p"], seed=3, offset=4)
    _check(got, idx, gap, margin, str(setting))


@pytest.mark.parametrize("V", [3000, 20000])
def test_filtered_special_rows(dev, V):
    B = 12
    x = synthetic.logits(B, V, seed=70)
    x[0, :] = -float("inf")                      # nothing valid
    x[1, ::2] = float("nan")
    x[2, 10] = x[2, 2000] = float("inf")         # +inf holds all the mass
    x[3, 100:200] = x[3].max() + 1.0             # a tie class at the top
    x[4, :] = 0.5                                 # every logit equal
    t = synthetic.temperatures(B, seed=71)
    t[5], t[6], t[7] = 0.0, -2.0, float("nan")   # greedy
    t[8] = float("inf")                           # uniform over the valid tokens
    k = torch.full((B,), 20, dtype=torch.int32)
    p = torch.full((B,), 0.8)
    m = torch.full((B,), 0.1)
    for fp64 in (False, True):
        got = _run(dev, x, t, k, p, m, seed=8, offset=9, fp64=fp64)
        idx, gap, margin = _oracle(x, t, k, p, m, seed=8, offset=9, fp64=fp64)
        _check(got, idx, gap, margin, f"special rows fp64={fp64}")
        assert got[0] == -1 and got[2] == 10
        assert 100 <= got[3] < 200
        assert got[5] == int(np.nanargmax(x[5].numpy()))


@pytest.mark.parametrize("fp64", [False, True])
def test_filtered_many_candidates(dev, fp64):
    """Rows where more tokens than the LDS holds can be kept: large tie classes
    (which top-p and min-p keep or drop whole, far from their boundaries), an
    infinite temperature, a top-k beyond the LDS capacity on nearly flat rows;
    ordinary rows in the same launch."""
    B, V = 10, 50000
    say(f"filtered rows with many candidates fp64={fp64}")
    g = torch.Generator().manual_seed(120)
    x = torch.randn((B, V), generator=g) - 10.0
    x[0, :20000] = 1.0                               # a tie class of 20000
    x[2] = torch.randn((V,), generator=g) * 0.05     # nearly flat
    x[3] = torch.randn((V,), generator=g) * 0.05
    x[4, 5000:17000] = 2.0                           # a tie class of 12000
    x[5, :9000] = 0.0                                # two close tie classes of 9000
    x[5, 9000:18000] = -0.001
    x[6:] = synthetic.logits(B - 6, V, seed=121)     # ordinary rows
    t = synthetic.temperatures(B, seed=122)
    t[1] = float("inf")
    k = torch.tensor([0, 30000, 9000, 20000, 0, 0, 100, 0, 50, 0], dtype=torch.int32)
    p = torch.tensor([0.9, 1.0, 1.0, 1.0, 1.0, 0.5, 1.0, 0.9, 0.95, 1.0])
    m = torch.tensor([0.0, 0.0, 0.0, 0.5, 0.5, 0.0, 0.1, 0.0, 0.05, 0.2])
    got = _run(dev, x, t, k, p, m, seed=12, offset=13, fp64=fp64)
    idx, gap, margin = _oracle(x, t, k, p, m, seed=12, offset=13, fp64=fp64)
    assert (margin[:6] > MARGIN).all(), margin
    _check(got, idx, gap, margin, f"many candidates fp64={fp64}")
    assert got[0] < 20000 and 5000 <= got[4] < 17000 and got[5] < 9000


@pytest.mark.parametrize("V", [3000, 20000])
def test_filtered_adjacent_floats(dev, V):
    """The 100 largest logits are consecutive float32 values above 5: the
    selections must resolve keys that differ only in their last bits."""
    B = 4
    x = synthetic.logits(B, V, std=1.0, seed=130) - 5.0
    chain = np.nextafter(np.float32(5.0), np.float32(np.inf)) * np.ones(100, dtype=np.float32)
    for j in range(1, 100):
        chain[j] = np.nextafter(chain[j - 1], np.float32(np.inf))
    for r in range(B):
        x[r, torch.randperm(V, generator=torch.Generator().manual_seed(131 + r))[:100]] = \
            torch.from_numpy(chain)
    t = torch.full((B,), 0.9)
    k = torch.tensor([37, 1, 0, 99], dtype=torch.int32)
    p = torch.tensor([1.0, 1.0, 0.5, 0.3])
    for fp64 in (False, True):
        got = _run(dev, x, t, k, p, None, seed=14, offset=15, fp64=fp64)
        idx, gap, margin = _oracle(x, t, k, p, None, seed=14, offset=15, fp64=fp64)
        _check(got, idx, gap, margin, f"adjacent floats V={V} fp64={fp64}")


@pytest.mark.parametrize("V", [7001, 40000])
def test_filters_off_equals_unfiltered(dev, V):
    B = 40
    x = synthetic.logits(B, V, seed=80)
    x[1, 5] = float("nan")
    x[2, :] = -float("inf")
    t = synthetic.temperatures(B, seed=81)
    t[3] = 0.0
    dx, dt = x.to(dev), t.to(dev)
    off_k = torch.zeros(B, dtype=torch.int32, device=dev)
    off_p = torch.full((B,), 1.0, device=dev)
    for fp64 in (False, True):
        a = fs.sample_logits(dx, dt, seed=11, offset=12, fp64_noise=fp64)
        b = fs.sample_logits_filtered(dx, dt, seed=11, offset=12, fp64_noise=fp64)
        c = fs.sample_logits_filtered(dx, dt, top_k=off_k, top_p=off_p, seed=11, offset=12,
                                      fp64_noise=fp64)
        assert torch.equal(a, b) and torch.equal(a, c)


def test_draws_stay_in_the_kept_set(dev):
    B, V = 32, 20000
    x = synthetic.logits(B, V, seed=90)
    t = synthetic.temperatures(B, seed=91)
    k, p, m = synthetic.filter_settings(B, V, seed=92)
    kept, margin = oracle.filter_kept(x.numpy(), t.numpy(), top_k=k.numpy(), top_p=p.numpy(),
                                      min_p=m.numpy())
    sure = margin > MARGIN
    dx, dt, dk, dp, dm = (v.to(dev) for v in (x, t, k, p, m))
    outs = torch.stack([fs.sample_logits_filtered(dx, dt, top_k=dk, top_p=dp, min_p=dm, seed=5,
                                                  offset=o) for o in range(200)]).cpu().numpy()
    for b in np.flatnonzero(sure):
        assert kept[b, outs[:, b]].all(), f"row {b} drew outside its kept set"
    # replays are bitwise reproducible
    again = fs.sample_logits_filtered(dx, dt, top_k=dk, top_p=dp, min_p=dm, seed=5, offset=3)
    assert np.array_equal(again.cpu().numpy(), outs[3])


@pytest.mark.parametrize("fp64", [False, True])
def test_filtered_law_chi_square(dev, fp64):
    row = torch.tensor([2.0, 1.6, 1.5, 1.0, 0.9, 0.2, -0.3, -1.0, 0.7, 1.55])
    t, k, p, m = 0.8, 7, 0.85, 0.08
    n = 262144
    x = row[None].repeat(n, 1)
    kept, margin = oracle.filter_kept(row[None].numpy(), np.array([t], dtype=np.float32), top_k=k,
                                      top_p=p, min_p=m)
    assert margin[0] > MARGIN
    z = row.double().numpy() / t
    law = np.where(kept[0], np.exp(z - z.max()), 0.0)
    law /= law.sum()
    got = fs.sample_logits_filtered(x.to(dev), t, top_k=k, top_p=p, min_p=m, seed=21, offset=0,
                                    row_ids=synthetic.row_ids(n).to(dev), fp64_noise=fp64)
    counts = np.bincount(got.cpu().numpy(), minlength=row.numel())
    assert counts[~kept[0]].sum() == 0
    keep = np.flatnonzero(kept[0])
    chi2 = stats.chi2_statistic(counts[keep], law[keep])
    say(f"  filtered chi2 = {chi2:.2f} (dof {keep.size - 1})")
    assert chi2 < stats.chi2_quantile(keep.size - 1, 1e-6)


@pytest.mark.parametrize("B", [8, 64])
def test_filtered_qwen_vocabulary(dev, B):
    V = 151936
    say(f"filtered parity at B={B} V={V}")
    x = synthetic.logits(B, V, seed=100)
    t = synthetic.temperatures(B, seed=101)
    k, p, m = synthetic.filter_settings(B, V, seed=102)
    for fp64 in (False, True):
        got = _run(dev, x, t, k, p, m, seed=1234, offset=17, fp64=fp64)
        idx, gap, margin = _oracle(x, t, k, p, m, seed=1234, offset=17, fp64=fp64)
        _check(got, idx, gap, margin, f"qwen vocabulary fp64={fp64}")
