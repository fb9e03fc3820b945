"""The workspace contract of the C ABI, on the GPU.

Stage 2 runs in the last workgroup of each batch tile (fused) or row
(standalone), chosen by completion counters in a fixed region at the start of
the workspace.  The caller zero-fills the workspace once; every call must leave
the counters zero again, so one workspace serves calls of any shape in turn.
The standalone sampler splits batches beyond the counter region over several
launches, which must not change any row's draw.
"""
import numpy as np
import pytest
import torch

import decode_exact_categorical_amd as fs
import oracle
import synthetic
from gpu_common import check_index_parity, need_gpu, say

pytestmark = pytest.mark.gpu

COUNTER_BYTES = 65536 * 4


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _fused(lib, H, W, temp, ws, seed, offset, fp64):
    B, D = H.shape
    V = W.shape[0]
    out = torch.full((B,), -7, dtype=torch.int64, device=H.device)
    st = lib.fs_sample_fused(fs._ptr(H), fs._ptr(W), B, D, V, fs._ptr(temp), None, seed, offset,
                             fs._ptr(out), None, fs.FS_FP64_NOISE if fp64 else 0, fs._ptr(ws),
                             ws.numel(), fs._stream(H.device))
    assert st == 0, lib.fs_last_error()
    return out


def _logits(lib, X, temp, ws, seed, offset, fp64, row_ids=None):
    B, V = X.shape
    out = torch.full((B,), -7, dtype=torch.int64, device=X.device)
    st = lib.fs_sample_logits(fs._ptr(X), B, V, fs._ptr(temp), seed, offset, int(fp64),
                              fs._ptr(out), fs._ptr(row_ids), fs._ptr(ws), ws.numel(),
                              fs._stream(X.device))
    assert st == 0, lib.fs_last_error()
    return out


def test_one_workspace_serves_every_shape(dev):
    """Calls of different kinds and shapes, in turn, on one workspace give the
    draws each gives on a fresh workspace, and leave the counters zero."""
    lib = fs.load_library()
    g = torch.Generator(device="cpu").manual_seed(7)
    cases = []
    for (kind, B, D, V, fp64) in [("fused", 64, 512, 32768, False),
                                  ("logits", 300, 0, 5000, True),
                                  ("fused", 1, 256, 70000, True),
                                  ("fused", 130, 128, 1000, False),
                                  ("logits", 3, 0, 10, False),
                                  ("logits", 4096, 0, 2048, False)]:
        temp = (0.5 + torch.rand(B, generator=g)).to(dev)
        if kind == "fused":
            args = (synthetic.hidden(B, D, seed=B).to(dev),
                    synthetic.weight(V, D, std=0.05, seed=V).to(dev), temp)
        else:
            args = (torch.randn(B, V, generator=g).to(dev), temp)
        need = lib.fs_workspace_bytes(B, V, fs.FS_FP64_NOISE if fp64 else 0)
        cases.append((kind, B, V, fp64, args, need))
    size = max(c[5] for c in cases)
    assert size > COUNTER_BYTES

    def run(c, ws, offset):
        kind, B, V, fp64, args, _ = c
        if kind == "fused":
            return _fused(lib, *args, ws, 31, offset, fp64)
        return _logits(lib, *args, ws, 31, offset, fp64)

    refs = []
    for i, c in enumerate(cases):
        say(f"fresh workspace: {c[0]} B={c[1]} V={c[2]} fp64={c[3]}")
        refs.append(run(c, torch.zeros(c[5], dtype=torch.uint8, device=dev), 100 + i).cpu())
    torch.cuda.synchronize()
    shared = torch.zeros(size, dtype=torch.uint8, device=dev)
    for rep in range(3):
        for i, c in enumerate(cases):
            say(f"shared workspace, round {rep}: {c[0]} B={c[1]} V={c[2]} fp64={c[3]}")
            got = run(c, shared, 100 + i).cpu()
            assert torch.equal(got, refs[i]), f"case {i} differs on the shared workspace"
            assert (got >= 0).all()
    torch.cuda.synchronize()
    assert int(shared[:COUNTER_BYTES].count_nonzero()) == 0, "counters not left at zero"


def test_logits_batch_beyond_one_launch(dev):
    """More rows than the counter region: split over launches, default row ids
    continue across them, and sampled rows match the oracle."""
    lib = fs.load_library()
    B, V = 65536 + 1500, 24
    g = torch.Generator(device="cpu").manual_seed(8)
    X = torch.randn(B, V, generator=g) * 2.0
    temp = torch.full((B,), 0.9)
    Xd, Td = X.to(dev), temp.to(dev)
    ws = torch.zeros(lib.fs_workspace_bytes(B, V, 0), dtype=torch.uint8, device=dev)
    say(f"standalone B={B} V={V}, default row ids")
    a = _logits(lib, Xd, Td, ws, 5, 77, False)
    ids = torch.arange(B, dtype=torch.int32, device=dev)
    say(f"standalone B={B} V={V}, explicit row ids 0..B-1")
    b = _logits(lib, Xd, Td, ws, 5, 77, False, row_ids=ids)
    torch.cuda.synchronize()
    a, b = a.cpu().numpy(), b.cpu().numpy()
    np.testing.assert_array_equal(a, b)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 65535, 65536, B - 1], rng.integers(0, B, 60)]))
    ref, gap, _ = oracle.sample_logits(X.numpy()[rows], temp.numpy()[rows], seed=5, offset=77,
                                       row_ids=rows.astype(np.uint32))
    check_index_parity(a[rows], ref, gap, f"standalone B={B} sampled rows")
    assert int(ws[:COUNTER_BYTES].count_nonzero()) == 0


def test_one_workspace_serves_every_entry_point(dev):
    """The binding keeps one cached workspace per stream for every entry point.
    Split-row filtered sampling and verification write their chunk data after
    the counter region, never inside it, so the standalone sampler's per-row
    counters (here 200 rows: past the first 256 bytes) and the fused sampler's
    stay zero whatever ran before them."""
    say("filtered (split rows) -> verify -> standalone B=200 -> fused, one workspace")
    B, V = 200, 20000
    X = synthetic.logits(B, V, seed=80)
    t = synthetic.temperatures(B, seed=81)
    Xd, td = X.to(dev), t.to(dev)
    fs.sample_logits_filtered(Xd[:8].contiguous(), td[:8].contiguous(), top_k=50, top_p=0.9,
                              seed=1, offset=2)          # split rows, one launch
    fs.sample_logits_filtered(Xd[:40].contiguous(), td[:40].contiguous(), top_p=0.9, seed=1,
                              offset=2)                  # split rows, two launches
    tg, dr, tok = synthetic.spec_decode(4, 2, V, seed=82)
    fs.verify(tg.to(dev), dr.to(dev), tok.to(dev), td[:4].contiguous(), seed=3, offset=4)
    got = fs.sample_logits(Xd, td, seed=5, offset=6)
    torch.cuda.synchronize()
    ref, gap, _ = oracle.sample_logits(X.numpy(), t.numpy(), seed=5, offset=6)
    check_index_parity(got.cpu().numpy(), ref, gap, "standalone after the other entry points")
    H = synthetic.hidden(70, 512, seed=83)
    W = synthetic.weight(3000, 512, std=0.3, seed=84)
    t2 = synthetic.temperatures(70, seed=85)
    got = fs.sample_fused(H.to(dev), W.to(dev), t2.to(dev), seed=7, offset=8)
    torch.cuda.synchronize()
    ref, gap, _ = oracle.sample_fused(H, W, t2.numpy(), seed=7, offset=8)
    check_index_parity(got.cpu().numpy(), ref, gap, "fused after the other entry points")


def test_fused_filtered_shares_the_workspace(dev):
    """The fused filtered sampler keeps its fallback flags in the counter region
    (word 0 their count, words 1 .. B the rows') and its records and fallback
    logits after it: after it runs (fallback rows included) the counters are
    zero and the other entry points draw what the oracle draws; and after them
    it still matches the materialised path."""
    say("fused filtered (with fallback rows) -> fused -> fused filtered, one workspace")
    B, D, V = 12, 256, 6000
    H = synthetic.hidden(B, D, seed=90)
    W = synthetic.weight(V, D, std=0.004, seed=91)       # flat rows: top-p alone falls back
    t = torch.full((B,), 1.0)
    Hd, Wd, td = H.to(dev), W.to(dev), t.to(dev)
    fs.sample_fused_filtered(Hd, Wd, td, top_p=0.9, seed=1, offset=1)
    torch.cuda.synchronize()
    ws = fs._workspace(dev, 0)
    assert int(ws[:4 * (B + 1)].view(torch.int32).abs().sum().item()) == 0
    t2 = synthetic.temperatures(B, seed=92)
    got = fs.sample_fused(Hd, Wd, t2.to(dev), seed=7, offset=8)
    torch.cuda.synchronize()
    ref, gap, _ = oracle.sample_fused(H, W, t2.numpy(), seed=7, offset=8)
    check_index_parity(got.cpu().numpy(), ref, gap, "fused after the fused filtered sampler")
    a = fs.sample_fused_filtered(Hd, Wd, td, top_p=0.9, seed=2, offset=3)
    Y = fs.debug_logits(Hd, Wd)
    b = fs.sample_logits_filtered(Y, td, top_p=0.9, seed=2, offset=3)
    assert torch.equal(a, b)
