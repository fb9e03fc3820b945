"""GPU parity at the full LM-head sizes, in the launch configuration the benchmark
times (the C ABI's fused entry point on torch's current stream).

* Qwen3-8B-shaped head: D = 4096, V = 151936, B in {1, 8, 32, 64}, per-row
  temperatures ~ U[0.5, 1.2], seeded per row.  The oracle computes all 64 rows.
* Llama-3-shaped head at the compute crossover: D = 4096, V = 128256, B = 256,
  fp32 bias ~ N(0, 1) with 10% of each row masked to -inf; oracle on 8 sampled rows.
* Wide head: D = 8192, V = 262144, B in {1, 16, 128}, T = 0.7, float64 noise;
  oracle on sampled rows; batch-permutation invariance at B = 16.
* The 128-column tiles (B > 64) at both of those heads (B = 128 with float64
  noise, B = 256 with the bias and mask): non-default row ids (around 10^9)
  against the oracle on sampled rows, a batch permutation carried with its row
  ids bitwise equal to the unpermuted draws, and single-row calls equal to the
  batched draws on those rows (where the oracle's gap exceeds the parity gap:
  a single row runs 16-column tiles, whose k rotation differs, so its float32
  logits may differ in the last bits).
"""
import numpy as np
import pytest
import torch

import decode_exact_categorical_amd as fs
import oracle
import synthetic
from gpu_common import GAP, LOGIT_TOL, check_index_parity, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


@pytest.fixture(scope="module")
def qwen_head(dev):
    say("generating the D=4096 V=151936 head")
    W = synthetic.weight(151936, 4096, std=0.02)
    H = synthetic.hidden(64, 4096)
    temp = synthetic.temperatures(64)
    return H, W, temp, W.to(dev)


def test_qwen_head_all_batches(dev, qwen_head):
    H, W, temp, Wd = qwen_head
    say("oracle: 64 rows at D=4096 V=151936")
    ref, gap, _ = oracle.sample_fused(H, W, temp.numpy(), seed=1234, offset=17)
    for B in (1, 8, 32, 64):
        say(f"fused B={B}")
        got = fs.sample_fused(H[:B].to(dev), Wd, temp[:B].to(dev), seed=1234, offset=17)
        torch.cuda.synchronize()
        check_index_parity(got.cpu().numpy(), ref[:B], gap[:B], f"qwen head B={B}")


def test_qwen_head_logits_sampled_rows(dev, qwen_head):
    H, W, _, Wd = qwen_head
    say("debug logits B=64 full V")
    Y = fs.debug_logits(H.to(dev), Wd)
    torch.cuda.synchronize()
    for r in (0, 63):
        ref = oracle.logits(H[r:r + 1], W)[0]
        err = np.abs(Y[r].cpu().double().numpy() - ref).max()
        say(f"  row {r}: max |dy| = {err:.3e}")
        assert err <= LOGIT_TOL


@pytest.fixture(scope="module")
def llama_head(dev):
    B, D, V = 256, 4096, 128256
    say("generating the D=4096 V=128256 head with bias")
    W = synthetic.weight(V, D, std=0.02)
    H = synthetic.hidden(B, D)
    temp = synthetic.temperatures(B)
    bias = synthetic.bias_with_mask(B, V, 0.1)
    return H, W, temp, bias, W.to(dev)


def test_llama_head_b256_bias_mask(dev, llama_head):
    H, W, temp, bias, Wd = llama_head
    B = H.shape[0]
    got = fs.sample_fused(H.to(dev), Wd, temp.to(dev), bias.to(dev), seed=1234, offset=3)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    rows = np.array([0, 1, 63, 64, 127, 128, 200, 255])
    say(f"oracle rows {rows.tolist()}")
    ref, gap, _ = oracle.sample_fused(H[rows], W, temp[rows].numpy(), bias[rows].numpy(),
                                      seed=1234, offset=3, row_ids=rows.astype(np.uint32))
    check_index_parity(got[rows], ref, gap, "llama head B=256")
    assert np.all(np.isfinite(bias[np.arange(B), got].numpy()))      # never a masked token


@pytest.fixture(scope="module")
def wide_head(dev):
    D, V = 8192, 262144
    say("generating the D=8192 V=262144 head (4 GiB)")
    W = synthetic.weight(V, D, std=0.015)
    H = synthetic.hidden(128, D)
    return H, W, W.to(dev)


def test_wide_head_fp64_noise(dev, wide_head):
    H, W, Wd = wide_head
    temp = torch.full((128,), 0.7)
    rows = np.array([0, 5, 15, 77, 127])
    say(f"oracle rows {rows.tolist()} at D=8192 V=262144")
    ref, gap, _ = oracle.sample_fused(H[rows], W, temp[rows].numpy(), seed=99, offset=123,
                                      row_ids=rows.astype(np.uint32), fp64_noise=True)
    for B in (1, 16, 128):
        say(f"fused fp64 B={B}")
        got = fs.sample_fused(H[:B].to(dev), Wd, temp[:B].to(dev), seed=99, offset=123,
                              fp64_noise=True)
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        sel = rows[rows < B]
        check_index_parity(got[sel], ref[:len(sel)], gap[:len(sel)], f"wide head B={B}")
        if B == 16:
            Hd = H[:16].to(dev)
            perm = torch.randperm(16, generator=torch.Generator().manual_seed(2))
            ids = torch.arange(16, dtype=torch.int32)[perm]
            p = fs.sample_fused(Hd[perm.to(dev)].contiguous(), Wd, temp[:16].to(dev), seed=99,
                                offset=123, row_ids=ids.to(dev), fp64_noise=True)
            assert np.array_equal(p.cpu().numpy(), got[perm.numpy()])


def _wide_tile_checks(dev, H, W, Wd, temp, bias, *, seed, offset, fp64, rows, singles, what):
    """Row ids around 10^9 against the oracle on `rows`; a permutation carried
    with its ids, bitwise; single-row calls on `singles` against the batch."""
    B = H.shape[0]
    ids = (10**9 + 7 * np.arange(B)).astype(np.uint32)
    Hd, td = H.to(dev), temp.to(dev)
    bd = None if bias is None else bias.to(dev)
    idd = torch.from_numpy(ids.view(np.int32)).to(dev)
    say(f"{what}: B={B} with row ids 10^9 + 7b")
    got = fs.sample_fused(Hd, Wd, td, bd, seed=seed, offset=offset, row_ids=idd,
                          fp64_noise=fp64).cpu().numpy()
    say(f"  oracle rows {rows.tolist()}")
    ref, gap, _ = oracle.sample_fused(H[rows], W, temp[rows].numpy(),
                                      None if bias is None else bias[rows].numpy(), seed=seed,
                                      offset=offset, row_ids=ids[rows], fp64_noise=fp64)
    check_index_parity(got[rows], ref, gap, f"{what} ids 10^9")
    say("  permuted batch with its ids")
    perm = torch.randperm(B, generator=torch.Generator().manual_seed(5))
    pd = perm.to(dev)
    p = fs.sample_fused(Hd[pd].contiguous(), Wd, td[pd].contiguous(),
                        None if bd is None else bd[pd].contiguous(), seed=seed, offset=offset,
                        row_ids=idd[pd].contiguous(), fp64_noise=fp64).cpu().numpy()
    assert np.array_equal(p, got[perm.numpy()]), f"{what}: permuted draws differ"
    compared = 0
    for r in singles:
        say(f"  single row {r}")
        s1 = fs.sample_fused(Hd[r:r + 1].contiguous(), Wd, td[r:r + 1].contiguous(),
                             None if bd is None else bd[r:r + 1].contiguous(), seed=seed,
                             offset=offset, row_ids=idd[r:r + 1].contiguous(),
                             fp64_noise=fp64).item()
        j = int(np.flatnonzero(rows == r)[0])
        if gap[j] > GAP:
            assert s1 == got[r] == ref[j], (what, r, s1, got[r], ref[j])
            compared += 1
    assert compared >= len(singles) - 1, f"{what}: single-row checks all near ties"


def test_wide_tiles_wide_head_b128(dev, wide_head):
    H, W, Wd = wide_head
    temp = torch.full((128,), 0.7)
    _wide_tile_checks(dev, H, W, Wd, temp, None, seed=41, offset=2**40 + 9, fp64=True,
                      rows=np.array([0, 33, 64, 100, 127]), singles=(0, 64, 127),
                      what="wide head fp64")


def test_wide_tiles_llama_head_b256(dev, llama_head):
    H, W, temp, bias, Wd = llama_head
    _wide_tile_checks(dev, H, W, Wd, temp, bias, seed=42, offset=77, fp64=False,
                      rows=np.array([1, 90, 128, 191, 254]), singles=(1, 128, 254),
                      what="llama head bias")
