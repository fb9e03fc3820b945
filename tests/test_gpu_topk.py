"""Gumbel-top-k on the GPU against the oracle, through the C ABI.

Parity rule for places: place j of a row must equal the oracle's wherever the
oracle's scores around it are separated by more than 1e-3 on both sides
(s_(j-1) - s_(j) and s_(j) - s_(j+1)); elsewhere the place is counted.  Every
row must hold distinct valid indices, and -1 exactly where the oracle has no
valid score left.  Greedy rows are exact; the law is checked directly on the
GPU's draws by chi-square against the Plackett-Luce probabilities.
"""
import itertools

import numpy as np
import pytest
import torch
from scipy import stats

import decode_exact_categorical_amd as fs
import oracle
import synthetic
from gpu_common import GAP, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def check_places(got, ref_idx, ref_top, what):
    """Assert the place parity rule; return the number of undecided places."""
    got = np.asarray(got)
    B, k = ref_idx.shape
    assert got.shape == (B, k)
    np.testing.assert_array_equal(got == -1, ref_idx == -1, err_msg=f"{what}: -1 places differ")
    for b in range(B):
        v = got[b][got[b] >= 0]
        assert len(set(v.tolist())) == v.size, f"{what}: row {b} repeats an index"
    before = np.concatenate([np.full((B, 1), np.inf), ref_top[:, :k - 1] - ref_top[:, 1:k]], axis=1)
    after_ = ref_top[:, :k] - ref_top[:, 1:k + 1]
    valid = ref_idx >= 0
    decided = valid & (before > GAP) & (after_ > GAP)
    bad = np.argwhere(decided & (got != ref_idx))
    assert bad.size == 0, (f"{what}: {len(bad)} decided places differ, e.g. {bad[:4].tolist()}: "
                           f"got {got[tuple(bad[:4].T)]} oracle {ref_idx[tuple(bad[:4].T)]}")
    und = int((valid & ~decided).sum())
    say(f"  top-k {what}: {int(decided.sum())} decided places equal, {und} undecided, "
        f"{int((valid & ~decided & (got != ref_idx)).sum())} of them differ")
    return und


@pytest.mark.parametrize("fp64", [False, True])
@pytest.mark.parametrize("B,V,k,misalign", [(8, 131072, 8, False), (33, 1001, 4, False),
                                            (5, 4099, 8, True), (3, 5, 8, False),
                                            (300, 2048, 2, False), (2, 70000, 1, False)])
def test_logits_topk_parity(dev, B, V, k, misalign, fp64):
    say(f"logits top-k B={B} V={V} k={k} misalign={misalign} fp64={fp64}")
    g = torch.Generator().manual_seed(41)
    x = torch.randn((B, V), generator=g) * 3.0
    temp = synthetic.temperatures(B, seed=42)
    temp[0] = 0.0
    if misalign:
        buf = torch.empty(B * V + 1, dtype=torch.float32, device=dev)
        xd = buf[1:].view(B, V)
        xd.copy_(x.to(dev))
    else:
        xd = x.to(dev)
    rid = synthetic.row_ids(B, start=900)
    got = fs.sample_logits_topk(xd, temp.to(dev), k=k, seed=5, offset=77, row_ids=rid.to(dev),
                                fp64_noise=fp64)
    torch.cuda.synchronize()
    ref, top = oracle.sample_logits_topk(x.numpy(), temp.numpy(), k=k, seed=5, offset=77,
                                         row_ids=rid.numpy().view(np.uint32), fp64_noise=fp64)
    got = got.cpu().numpy()
    np.testing.assert_array_equal(got[0], ref[0])        # greedy row
    check_places(got, ref, top, f"B={B} V={V} k={k} fp64={fp64}")


def test_logits_topk_place0_is_the_single_draw(dev):
    """With float64 noise both kernels form (y / t) + g in float64: bitwise equal."""
    g = torch.Generator().manual_seed(43)
    x = (torch.randn((64, 20000), generator=g) * 2.0).to(dev)
    temp = synthetic.temperatures(64, seed=44).to(dev)
    a = fs.sample_logits_topk(x, temp, k=5, seed=8, offset=9, fp64_noise=True)
    b = fs.sample_logits(x, temp, seed=8, offset=9, fp64_noise=True)
    assert torch.equal(a[:, 0], b)


def test_logits_topk_masks_greedy_ties_and_short_rows(dev):
    rng = np.random.default_rng(6)
    V, k = 3000, 8
    x = rng.integers(-2, 2, size=(6, V)).astype(np.float32)
    x[1] = -np.inf
    x[1, [10, 2999, 500]] = [0.0, 1.0, 0.0]           # three valid entries
    x[2] = np.nan
    x[2, 7] = 3.0                                      # one valid entry
    x[3] = -np.inf                                     # none
    x[4, ::3] = -np.inf
    temp = np.array([0.0, 1.0, 0.7, 1.0, 0.0, -1.0], dtype=np.float32)
    got = fs.sample_logits_topk(torch.from_numpy(x).to(dev), torch.from_numpy(temp).to(dev), k=k,
                                seed=1, offset=2).cpu().numpy()
    ref, top = oracle.sample_logits_topk(x, temp, k=k, seed=1, offset=2)
    for b in (0, 4, 5):                                 # greedy rows with ties: exact
        np.testing.assert_array_equal(got[b], ref[b])
    assert sorted(got[1, :3].tolist()) == [10, 500, 2999] and (got[1, 3:] == -1).all()
    assert got[2, 0] == 7 and (got[2, 1:] == -1).all()
    assert (got[3] == -1).all()
    assert (got[4] % 3 != 0).all()
    check_places(got, ref, top, "masks")


@pytest.mark.parametrize("fp64", [False, True])
def test_logits_topk_law_on_gpu(dev, fp64):
    """Ordered places (i, j, l) of a 4-token row over 262144 logical rows follow
    sequential sampling without replacement from softmax (chi-square, 23 dof)."""
    y = torch.tensor([1.0, 0.5, 0.0, -0.7])
    t, n, k = 0.8, 262144, 3
    x = y.repeat(n, 1).to(dev)
    got = fs.sample_logits_topk(x, torch.full((n,), t, device=dev), k=k, seed=123, offset=4,
                                fp64_noise=fp64).cpu().numpy()
    assert (got >= 0).all() and (got < 4).all()
    p = np.exp(y.double().numpy() / t)
    p /= p.sum()
    seqs = list(itertools.permutations(range(4), k))
    expected = []
    for s in seqs:
        pr, left = 1.0, 1.0
        for i in s:
            pr *= p[i] / left
            left -= p[i]
        expected.append(pr)
    expected = np.array(expected)
    code = got[:, 0] * 16 + got[:, 1] * 4 + got[:, 2]
    counts = np.array([(code == s[0] * 16 + s[1] * 4 + s[2]).sum() for s in seqs], dtype=np.float64)
    assert counts.sum() == n
    chi2 = ((counts - n * expected) ** 2 / (n * expected)).sum()
    say(f"  chi2 = {chi2:.1f} over {len(seqs) - 1} dof")
    assert chi2 < stats.chi2.ppf(1 - 1e-6, len(seqs) - 1)


def test_topk_argument_errors(dev):
    lib = fs.load_library()
    x = torch.zeros((2, 10), device=dev)
    t = torch.ones(2, device=dev)
    out = torch.empty((2, 9), dtype=torch.int64, device=dev)
    ws = torch.zeros(lib.fs_workspace_bytes_topk(2, 10, 0), dtype=torch.uint8, device=dev)
    for k in (0, fs.FS_TOPK_MAX + 1):
        assert lib.fs_sample_logits_topk(fs._ptr(x), 2, 10, fs._ptr(t), 1, 1, 0, k, fs._ptr(out),
                                         None, fs._ptr(ws), ws.numel(), fs._stream(dev)) == 1
    small = torch.zeros(lib.fs_workspace_bytes(2, 10, 0), dtype=torch.uint8, device=dev)
    if small.numel() < ws.numel():
        assert lib.fs_sample_logits_topk(fs._ptr(x), 2, 10, fs._ptr(t), 1, 1, 0, 2, fs._ptr(out),
                                         None, fs._ptr(small), small.numel(),
                                         fs._stream(dev)) == 3


def _fused_case(B, D, V, *, bias=False, greedy_rows=(), seed_base=0, w_std=0.02):
    H = synthetic.hidden(B, D, seed=220 + seed_base)
    W = synthetic.weight(V, D, std=w_std, seed=221 + seed_base)
    temp = synthetic.temperatures(B, seed=222 + seed_base)
    for r in greedy_rows:
        temp[r] = [0.0, -1.0, float("nan")][r % 3]
    bb = synthetic.bias_with_mask(B, V, 0.1, seed=223 + seed_base) if bias else None
    return H, W, temp, bb


FUSED_TOPK_CASES = [
    dict(B=4, D=512, V=32768, k=8),
    dict(B=37, D=200, V=1001, k=4, bias=True, greedy_rows=(0, 5, 9)),
    dict(B=20, D=64, V=170001, k=8),            # two passes per wave
    dict(B=3, D=64, V=13, k=8, w_std=1.0),
    dict(B=33, D=256, V=4000, k=2, bias=True),   # 16-byte bias rows, a 48- or 64-column tile
    dict(B=64, D=256, V=3001, k=8, greedy_rows=(17,)),
    dict(B=100, D=128, V=2000, k=3, bias=True),  # two 64-column tiles
]


@pytest.mark.parametrize("fp64", [False, True])
@pytest.mark.parametrize("case", FUSED_TOPK_CASES)
def test_fused_topk_parity(dev, case, fp64):
    case = dict(case)
    B, D, V, k = case.pop("B"), case.pop("D"), case.pop("V"), case.pop("k")
    say(f"fused top-k B={B} D={D} V={V} k={k} fp64={fp64} {case}")
    H, W, temp, bias = _fused_case(B, D, V, **case)
    Hd, Wd, td, bd = to_dev(H, W, temp, bias, dev=dev)
    rid = synthetic.row_ids(B, start=40)
    got = fs.sample_fused_topk(Hd, Wd, td, bd, k=k, seed=1234, offset=5, row_ids=rid.to(dev),
                               fp64_noise=fp64)
    torch.cuda.synchronize()
    ref, top = oracle.sample_fused_topk(H, W, temp.numpy(), None if bias is None else bias.numpy(),
                                        k=k, seed=1234, offset=5,
                                        row_ids=rid.numpy().view(np.uint32), fp64_noise=fp64)
    check_places(got.cpu().numpy(), ref, top, f"fused B={B} V={V} k={k} fp64={fp64}")


def test_fused_topk_place0_is_the_fused_draw(dev):
    """Float64 noise: the same logits and score expression, so place 0 equals
    fs_sample_fused's draw bit for bit."""
    H, W, temp, bias = _fused_case(40, 256, 5000, bias=True, seed_base=7)
    Hd, Wd, td, bd = to_dev(H, W, temp, bias, dev=dev)
    a = fs.sample_fused_topk(Hd, Wd, td, bd, k=3, seed=11, offset=12, fp64_noise=True)
    b = fs.sample_fused(Hd, Wd, td, bd, seed=11, offset=12, fp64_noise=True)
    assert torch.equal(a[:, 0], b)


def test_fused_topk_masks(dev):
    B, D, V, k = 6, 64, 300, 8
    H, W, temp, _ = _fused_case(B, D, V, seed_base=8)
    bias = torch.zeros((B, V))
    bias[1] = float("-inf")
    bias[2] = float("-inf")
    bias[2, [7, 123, 299]] = 0.0
    bias[3, ::2] = float("-inf")
    temp[4] = 0.0
    Hd, Wd, td, bd = to_dev(H, W, temp, bias, dev=dev)
    got = fs.sample_fused_topk(Hd, Wd, td, bd, k=k, seed=3, offset=4).cpu().numpy()
    assert (got[1] == -1).all()
    assert sorted(got[2, :3].tolist()) == [7, 123, 299] and (got[2, 3:] == -1).all()
    assert (got[3] % 2 == 1).all()
    ref, top = oracle.sample_fused_topk(H, W, temp.numpy(), bias.numpy(), k=k, seed=3, offset=4)
    np.testing.assert_array_equal(got[4], ref[4])                   # greedy row
    check_places(got, ref, top, "fused masks")


def test_fused_topk_law_on_gpu(dev):
    """One-hot hidden rows pick logits [1, 0.5, 0, -0.75] out of W; the ordered
    places over 131072 logical rows follow sampling without replacement."""
    n, D, k, t = 131072, 16, 3, 0.8
    y = torch.tensor([1.0, 0.5, 0.0, -0.75])
    W = torch.zeros((4, D), dtype=torch.bfloat16)
    W[:, 0] = y.to(torch.bfloat16)
    H = torch.zeros((n, D), dtype=torch.bfloat16)
    H[:, 0] = 1.0
    got = fs.sample_fused_topk(H.to(dev), W.to(dev), torch.full((n,), t, device=dev), k=k, seed=99,
                               offset=6).cpu().numpy()
    assert (got >= 0).all() and (got < 4).all()
    p = np.exp(y.double().numpy() / t)
    p /= p.sum()
    seqs = list(itertools.permutations(range(4), k))
    expected = []
    for s in seqs:
        pr, left = 1.0, 1.0
        for i in s:
            pr *= p[i] / left
            left -= p[i]
        expected.append(pr)
    expected = np.array(expected)
    code = got[:, 0] * 16 + got[:, 1] * 4 + got[:, 2]
    counts = np.array([(code == s[0] * 16 + s[1] * 4 + s[2]).sum() for s in seqs], dtype=np.float64)
    chi2 = ((counts - n * expected) ** 2 / (n * expected)).sum()
    say(f"  fused chi2 = {chi2:.1f} over {len(seqs) - 1} dof")
    assert chi2 < stats.chi2.ppf(1 - 1e-6, len(seqs) - 1)
