"""The entry point that allocates nothing (fs_sample_fused_noalloc), through the
C ABI: its draws equal fs_sample_fused's (the workspace entry point, same
kernels) bit for bit, call after call on the shared built-in scratch, the
second call of each pair smaller than the first; sizes past the scratch are
refused on the host."""
import numpy as np
import pytest
import torch

import decode_exact_categorical_amd as fs
import oracle
import synthetic
from gpu_common import check_index_parity, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _inputs(B, D, V, *, bias, seed, dev):
    H = synthetic.hidden(B, D, seed=seed)
    W = synthetic.weight(V, D, std=0.05, seed=seed + 1)
    temp = synthetic.temperatures(B, seed=seed + 2)
    if B >= 3:
        temp[2] = 0.0                                   # a greedy row
    bb = synthetic.bias_with_mask(B, V, 0.1, seed=seed + 3) if bias else None
    return H, W, temp, bb, [None if t is None else t.to(dev) for t in (H, W, temp, bb)]


# (B, D, V, fp64 noise, bias): pairs of calls, the second smaller than the first
PAIRS = [
    ((300, 512, 40000, False, True), (17, 512, 40000, False, True)),
    ((1024, 256, 9001, True, False), (1, 256, 9001, True, False)),
    ((64, 1024, 151936, False, False), (8, 1024, 151936, False, False)),
    ((129, 768, 20003, True, True), (65, 768, 20003, True, True)),
]


@pytest.mark.parametrize("pair", PAIRS)
def test_noalloc_equals_workspace_entry_point(dev, pair):
    for i, (B, D, V, fp64, bias) in enumerate(pair):
        say(f"no-alloc call {i}: B={B} D={D} V={V} fp64={fp64} bias={bias}")
        H, W, temp, bb, (Hd, Wd, td, bd) = _inputs(B, D, V, bias=bias, seed=400 + B, dev=dev)
        rid = torch.arange(B, dtype=torch.int32, device=dev) * 3 + 11
        ref = fs.sample_fused(Hd, Wd, td, bd, seed=71, offset=5 + i, row_ids=rid, fp64_noise=fp64)
        out = torch.full((B,), -7, dtype=torch.int64, device=dev)
        got = fs.sample_fused_noalloc(Hd, Wd, td, bd, seed=71, offset=5 + i, row_ids=rid,
                                      fp64_noise=fp64, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, ref), (B, (got != ref).nonzero()[:5])
        # a second call on the same scratch replays bit for bit
        again = fs.sample_fused_noalloc(Hd, Wd, td, bd, seed=71, offset=5 + i, row_ids=rid,
                                        fp64_noise=fp64)
        assert torch.equal(again, ref)
        # and a few rows against the oracle
        rows = np.unique(np.minimum(np.array([0, 2, B // 2, B - 1]), B - 1))
        r_idx, r_gap, _ = oracle.sample_fused(H[rows], W, temp[rows].numpy(),
                                              None if bb is None else bb[rows].numpy(), seed=71,
                                              offset=5 + i,
                                              row_ids=(rows * 3 + 11).astype(np.uint32),
                                              fp64_noise=fp64)
        check_index_parity(got.cpu().numpy()[rows], r_idx, r_gap, f"no-alloc B={B}")


def test_noalloc_refuses_sizes_past_the_scratch(dev):
    B, D, V = 1025, 64, 1000
    H = torch.zeros((B, D), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((V, D), dtype=torch.bfloat16, device=dev)
    t = torch.ones(B, device=dev)
    with pytest.raises(fs.FSampleError, match="FS_ERR_UNSUPPORTED"):
        fs.sample_fused_noalloc(H, W, t, seed=0, offset=0)
    z = fs.sample_fused_noalloc(H[:0], W, t[:0], seed=0, offset=0)
    assert z.numel() == 0
