"""GPU parity against the oracle, through the C ABI (small and ragged shapes).

Rules (fixed by the benchmark spec of this path): Philox words bit-exact; fused
logits within 2e-3 of the oracle's float64 logits; sampled indices bit-exact on
every row whose oracle top-2 perturbed-score gap exceeds 1e-3 (closer rows are
counted); greedy over materialised logits bit-exact on every row.
"""
import numpy as np
import pytest
import torch

import decode_exact_categorical_amd as fs
import oracle
import synthetic
from gpu_common import LOGIT_TOL, check_index_parity, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


@pytest.mark.parametrize("seed,offset,B,n_ctr,ids", [
    (1234, 0, 4, 8192, None),
    (0, 0, 1, 1, None),
    (0xFFFFFFFFFFFFFFFF, 0xFFFFFFFFFFFFFFFF, 3, 100, [0xFFFFFFFF, 7, 2**31]),
    (0x0123456789ABCDEF, 987654321987, 64, 2049, "arange"),
])
def test_philox_words_bit_exact(dev, seed, offset, B, n_ctr, ids):
    say(f"philox words seed={seed} offset={offset} B={B} n_ctr={n_ctr}")
    rid_np = None
    rid = None
    if ids == "arange":
        rid_np = np.arange(1000, 1000 + B, dtype=np.uint32)
    elif ids is not None:
        rid_np = np.array(ids, dtype=np.uint32)
    if rid_np is not None:
        rid = torch.from_numpy(rid_np.view(np.int32)).to(dev)
    got = fs.debug_philox_words(seed, offset, B, n_ctr, row_ids=rid, device=dev)
    torch.cuda.synchronize()
    got = got.cpu().numpy().view(np.uint32)
    ref = oracle.philox_words(seed, offset, rid_np, B, n_ctr)
    np.testing.assert_array_equal(got, ref)


LOGIT_SHAPES = [
    (4, 512, 32768),      # the tiny fused configuration
    (37, 200, 1001),      # ragged B, D % 32 != 0, V % 16 != 0
    (70, 520, 777),       # two batch tiles
    (1, 8, 5),            # smaller than one MFMA tile in every dimension
    (16, 4096, 2000),     # full-width contraction
    (33, 64, 4099),       # three column blocks
]


@pytest.mark.parametrize("B,D,V", LOGIT_SHAPES)
def test_debug_logits_match_oracle(dev, B, D, V):
    say(f"debug logits B={B} D={D} V={V}")
    H = synthetic.hidden(B, D, seed=11)
    W = synthetic.weight(V, D, std=0.02 if D >= 512 else 0.3, seed=12)
    Hd, Wd = to_dev(H, W, dev=dev)
    Y = fs.debug_logits(Hd, Wd)
    torch.cuda.synchronize()
    ref = oracle.logits(H, W)
    err = np.abs(Y.cpu().double().numpy() - ref).max()
    say(f"  max |dy| = {err:.3e}")
    assert err <= LOGIT_TOL


def _case(B, D, V, *, bias=False, greedy_rows=(), seed_base=0, w_std=0.02):
    H = synthetic.hidden(B, D, seed=20 + seed_base)
    W = synthetic.weight(V, D, std=w_std, seed=21 + seed_base)
    temp = synthetic.temperatures(B, seed=22 + seed_base)
    for r in greedy_rows:
        temp[r] = [0.0, -1.0, float("nan")][r % 3]
    bb = synthetic.bias_with_mask(B, V, 0.1, seed=23 + seed_base) if bias else None
    return H, W, temp, bb


FUSED_CASES = [
    dict(B=4, D=512, V=32768),
    dict(B=37, D=200, V=1001, bias=True, greedy_rows=(0, 5, 9)),
    dict(B=70, D=520, V=777, bias=True),
    dict(B=16, D=4096, V=5000, greedy_rows=(3,)),
    dict(B=3, D=64, V=13, w_std=1.0),
    # every batch width of a tile (16 / 32 / 48 / 64 columns), with and without
    # a bias, D % 32 != 0 and ragged V
    dict(B=24, D=96, V=1500, bias=True),
    dict(B=48, D=128, V=2500, greedy_rows=(1,)),
    dict(B=64, D=264, V=3001),
    # more than 80 rows per wave: several passes over each wave's rows at
    # every width, the running bests merged across passes
    dict(B=64, D=64, V=170001, greedy_rows=(2, 40)),
    dict(B=20, D=64, V=170001, bias=True),
    # batch tiles of 128 columns (B > 64): one partial tile, two tiles with a
    # bias and a contraction shorter than the noise slots, a full-width D
    dict(B=100, D=256, V=5001, greedy_rows=(7,)),
    dict(B=200, D=160, V=3001, bias=True, greedy_rows=(130,)),
    dict(B=129, D=4096, V=2000),
    dict(B=72, D=128, V=4000, bias=True),       # 16-byte bias rows, wide tile
]


@pytest.mark.parametrize("fp64", [False, True])
@pytest.mark.parametrize("case", FUSED_CASES)
def test_fused_sampling_parity(dev, case, fp64):
    case = dict(case)
    B, D, V = case.pop("B"), case.pop("D"), case.pop("V")
    say(f"fused sample B={B} D={D} V={V} fp64={fp64} {case}")
    H, W, temp, bias = _case(B, D, V, **case)
    Hd, Wd, td, bd = to_dev(H, W, temp, bias, dev=dev)
    got = fs.sample_fused(Hd, Wd, td, bd, seed=1234, offset=5, fp64_noise=fp64)
    torch.cuda.synchronize()
    ref, gap, _ = oracle.sample_fused(H, W, temp.numpy(), None if bias is None else bias.numpy(),
                                      seed=1234, offset=5, fp64_noise=fp64)
    check_index_parity(got.cpu().numpy(), ref, gap, f"B={B} V={V} fp64={fp64}")


@pytest.mark.parametrize("fp64", [False, True])
@pytest.mark.parametrize("B,V,misalign", [(8, 131072, False), (33, 1001, False), (5, 4099, True),
                                          (1, 3, False), (300, 2048, False)])
def test_logits_sampling_parity(dev, B, V, misalign, fp64):
    say(f"logits sample B={B} V={V} misalign={misalign} fp64={fp64}")
    g = torch.Generator().manual_seed(31)
    x = torch.randn((B, V), generator=g) * 3.0
    temp = synthetic.temperatures(B, seed=32)
    temp[0] = 0.0
    if misalign:   # a row stride of V with V % 4 != 0 and a buffer offset by one float
        buf = torch.empty(B * V + 1, dtype=torch.float32, device=dev)
        xd = buf[1:].view(B, V)
        xd.copy_(x.to(dev))
    else:
        xd = x.to(dev)
    rid = synthetic.row_ids(B, start=500)
    got = fs.sample_logits(xd, temp.to(dev), seed=99, offset=2**40 + 3, row_ids=rid.to(dev),
                           fp64_noise=fp64)
    torch.cuda.synchronize()
    ref, gap, _ = oracle.sample_logits(x.numpy(), temp.numpy(), seed=99, offset=2**40 + 3,
                                       row_ids=rid.numpy().view(np.uint32), fp64_noise=fp64)
    got = got.cpu().numpy()
    assert got[0] == ref[0]                   # greedy row: exact, ties included
    check_index_parity(got, ref, gap, f"logits B={B} V={V} fp64={fp64}")


@pytest.mark.parametrize("fp64", [False, True])
def test_logits_draws_independent_of_chunking(dev, fp64):
    # The standalone sampler splits a row into chunks whose length follows the
    # batch size (2048 logits at B = 8, 32768 at B = 320 and V = 131072), and
    # each chunk skips the noise of logits its running best rules out.  The
    # draw is the exhaustive argmax either way: the same rows with the same
    # ids give the same tokens bit for bit in a batch of 320 and in batches
    # of 8.
    say(f"logits sampler chunking invariance fp64={fp64}")
    B, V = 320, 131072
    g = torch.Generator(device=dev).manual_seed(41)
    x = torch.randn((B, V), generator=g, device=dev) * 3.0
    temp = (0.5 + torch.rand(B, generator=g, device=dev))
    temp[3] = 0.0
    rid = torch.arange(7000, 7000 + B, dtype=torch.int32, device=dev)
    whole = fs.sample_logits(x, temp, seed=5, offset=11, row_ids=rid, fp64_noise=fp64)
    parts = torch.cat([fs.sample_logits(x[r:r + 8].contiguous(), temp[r:r + 8].contiguous(), seed=5,
                                        offset=11, row_ids=rid[r:r + 8].contiguous(), fp64_noise=fp64)
                       for r in range(0, B, 8)])
    torch.cuda.synchronize()
    assert torch.equal(whole.cpu(), parts.cpu())
    assert (whole >= 0).all()


def test_greedy_logits_exact_with_ties(dev):
    say("greedy logits with ties")
    rng = np.random.default_rng(5)
    x = rng.integers(-2, 2, size=(64, 5000)).astype(np.float32)
    x[3] = -np.inf
    x[4, :] = np.nan
    x[4, 4999] = 1.0
    temp = np.zeros(64, np.float32)
    temp[10:20] = -3.0
    got = fs.sample_logits(torch.from_numpy(x).to(dev), torch.from_numpy(temp).to(dev), seed=0,
                           offset=0).cpu().numpy()
    ref, _, _ = oracle.sample_logits(x, temp, seed=0, offset=0)
    np.testing.assert_array_equal(got, ref)
    assert got[3] == -1 and got[4] == 4999


@pytest.mark.parametrize("fp64", [False, True])
def test_no_token_rows_and_masks(dev, fp64):
    say(f"masked rows fp64={fp64}")
    B, D, V = 6, 64, 300
    H, W, temp, _ = _case(B, D, V, seed_base=40)
    bias = torch.zeros((B, V))
    bias[1] = float("-inf")                 # every token masked
    bias[2, :] = float("-inf")
    bias[2, 123] = 0.0                      # a single survivor
    bias[3, ::2] = float("-inf")
    temp[4] = 0.0
    bias[4] = float("-inf")                 # masked greedy row
    Hd, Wd, td, bd = to_dev(H, W, temp, bias, dev=dev)
    got = fs.sample_fused(Hd, Wd, td, bd, seed=7, offset=1, fp64_noise=fp64).cpu().numpy()
    assert got[1] == -1 and got[2] == 123 and got[3] % 2 == 1 and got[4] == -1
    ref, gap, _ = oracle.sample_fused(H, W, temp.numpy(), bias.numpy(), seed=7, offset=1,
                                      fp64_noise=fp64)
    check_index_parity(got, ref, gap, "masked rows")


def test_empty_batch(dev):
    H = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((10, 64), dtype=torch.bfloat16, device=dev)
    assert fs.sample_fused(H, W, torch.empty(0, device=dev), seed=0, offset=0).numel() == 0
    x = torch.empty((0, 10), device=dev)
    assert fs.sample_logits(x, torch.empty(0, device=dev), seed=0, offset=0).numel() == 0


@pytest.mark.parametrize("fp64", [False, True])
def test_fused_replay_permutation_and_single_row(dev, fp64):
    """Seeded draws depend only on (seed, offset, row id): they replay bitwise, follow
    their rows under a batch permutation, and equal single-row calls."""
    say(f"fused invariance fp64={fp64}")
    B, D, V = 40, 256, 3001
    H, W, temp, bias = _case(B, D, V, bias=True, seed_base=50)
    Hd, Wd, td, bd = to_dev(H, W, temp, bias, dev=dev)
    rid = torch.arange(7, 7 + B, dtype=torch.int32, device=dev)
    a = fs.sample_fused(Hd, Wd, td, bd, seed=3, offset=11, row_ids=rid, fp64_noise=fp64).clone()
    b = fs.sample_fused(Hd, Wd, td, bd, seed=3, offset=11, row_ids=rid, fp64_noise=fp64)
    assert torch.equal(a, b)
    perm = torch.randperm(B, generator=torch.Generator().manual_seed(1)).to(dev)
    p = fs.sample_fused(Hd[perm].contiguous(), Wd, td[perm].contiguous(), bd[perm].contiguous(),
                        seed=3, offset=11, row_ids=rid[perm].contiguous(), fp64_noise=fp64)
    assert torch.equal(p, a[perm])
    for r in (0, 17, 39):
        s = fs.sample_fused(Hd[r:r + 1].contiguous(), Wd, td[r:r + 1].contiguous(),
                            bd[r:r + 1].contiguous(), seed=3, offset=11,
                            row_ids=rid[r:r + 1].contiguous(), fp64_noise=fp64)
        assert s.item() == a[r].item()
    o = fs.sample_fused(Hd, Wd, td, bd, seed=3, offset=12, row_ids=rid, fp64_noise=fp64)
    assert (o != a).sum().item() > B // 2


def test_replay_under_side_stream_contention(dev):
    """Bitwise replay while another stream runs a large matmul."""
    say("replay under contention")
    B, D, V = 64, 1024, 50000
    H, W, temp, _ = _case(B, D, V, seed_base=60)
    Hd, Wd, td = to_dev(H, W, temp, dev=dev)
    ref = fs.sample_fused(Hd, Wd, td, seed=9, offset=4).clone()
    big = torch.randn((4096, 4096), device=dev)
    side = torch.cuda.Stream(dev)
    mine = torch.cuda.Stream(dev)
    torch.cuda.synchronize()
    outs = []
    with torch.cuda.stream(side):
        for _ in range(8):
            big = big @ big
            big = big / big.norm()
    with torch.cuda.stream(mine):
        for _ in range(8):
            outs.append(fs.sample_fused(Hd, Wd, td, seed=9, offset=4).clone())
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)


def test_fused_matches_logits_sampler_stream(dev):
    """Same y + bias, same draws: the standalone sampler over the fused path's own
    logits draws from the same Philox stream.  With float64 noise both form the
    score as (y + bias) / t + g in float64, so they agree bitwise.  With float32
    noise the fused kernel folds t * g into the accumulator, so the scores differ
    by fp32 rounding and the draws agree on every row the oracle decides."""
    say("fused vs standalone on the same logits")
    B, D, V = 24, 512, 4096
    H, W, temp, _ = _case(B, D, V, seed_base=70)
    Hd, Wd, td = to_dev(H, W, temp, dev=dev)
    y = fs.debug_logits(Hd, Wd)
    a = fs.sample_fused(Hd, Wd, td, seed=5, offset=6, fp64_noise=True)
    b = fs.sample_logits(y, td, seed=5, offset=6, fp64_noise=True)
    assert torch.equal(a, b)
    a = fs.sample_fused(Hd, Wd, td, seed=5, offset=6).cpu().numpy()
    b = fs.sample_logits(y, td, seed=5, offset=6).cpu().numpy()
    ref, gap, _ = oracle.sample_logits(y.cpu().numpy(), temp.numpy(), seed=5, offset=6)
    check_index_parity(b, ref, gap, "standalone on fused logits")
    check_index_parity(a, ref, gap, "fused vs oracle on fused logits")


def test_noise_transform_float32_full_grid(dev):
    """The float32 E and g of every one of the 2^23 grid points, against the
    oracle's float64 values: E to a few float32 ulps relative (including the
    deep tail, u near 1), g to a few float32 ulps of max(1, |g|)."""
    say("noise transform: all 2^23 float32 grid points")
    k = np.arange(2**23, dtype=np.uint64)
    low = np.random.default_rng(3).integers(0, 512, size=k.size, dtype=np.uint64)
    words = ((k << np.uint64(9)) | low).astype(np.uint32)
    E, g = fs.debug_noise(torch.from_numpy(words.view(np.int32)).to(dev))
    E, g = E.cpu().numpy(), g.cpu().numpy()
    Eo, go = oracle.noise_grid(False, 0, 2**23)
    relE = np.abs(E - Eo) / Eo
    errg = np.abs(g - go) / np.maximum(1.0, np.abs(go))
    say(f"  max rel err E = {relE.max():.3e} (at u index {relE.argmax()}), "
        f"max err g / max(1,|g|) = {errg.max():.3e}")
    assert relE.max() <= NOISE32_E_REL and errg.max() <= NOISE32_G_REL


def test_noise_transform_float64_samples(dev):
    """Float64 noise on 64 runs of 16384 consecutive points of the 52-bit grid at
    random places plus both ends: E keeps float64 relative accuracy where
    u >= 1/2 (E < ln 2, the tail), float32 accuracy elsewhere; g is float32-accurate."""
    say("noise transform: float64 grid samples")
    rng = np.random.default_rng(4)
    starts = [0, 2**52 - 16384, 2**51 - 8192] + [int(x) for x in
                                                 rng.integers(0, 2**52 - 16384, size=61)]
    ks, Eo, go = [], [], []
    for k0 in starts:
        e, gg = oracle.noise_grid(True, k0, 16384)
        ks.append(np.arange(k0, k0 + 16384, dtype=np.uint64))
        Eo.append(e)
        go.append(gg)
    k = np.concatenate(ks)
    Eo, go = np.concatenate(Eo), np.concatenate(go)
    low = rng.integers(0, 4096, size=k.size, dtype=np.uint64)
    full = (k << np.uint64(12)) | low
    words = np.empty(2 * k.size, dtype=np.uint32)
    words[0::2] = (full >> np.uint64(32)).astype(np.uint32)
    words[1::2] = (full & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    E, g = fs.debug_noise(torch.from_numpy(words.view(np.int32)).to(dev), fp64_noise=True)
    E, g = E.cpu().numpy(), g.cpu().numpy()
    relE = np.abs(E - Eo) / Eo
    tail = Eo < np.log(2.0)
    errg = np.abs(g - go) / np.maximum(1.0, np.abs(go))
    say(f"  max rel err E: tail {relE[tail].max():.3e}, body {relE[~tail].max():.3e}; "
        f"max err g / max(1,|g|) = {errg.max():.3e}; E range [{E.min():.4e}, {E.max():.4f}]")
    assert relE[tail].max() <= NOISE64_E_TAIL_REL
    assert relE[~tail].max() <= NOISE32_E_REL
    assert errg.max() <= NOISE32_G_REL
    assert E.min() == pytest.approx(1.1102230246251565e-16, rel=1e-12)


# Bounds for the noise transforms (float32 unit roundoff u32 = 2^-24 ~ 6e-8):
# E is a handful of float32 operations (reciprocal, 8-term series or hardware
# log2, scaling), g one hardware log2 and one scaling; float64 E in the tail
# is a float64 division and a 16-term series.
NOISE32_E_REL = 8 * 2.0**-24
NOISE32_G_REL = 8 * 2.0**-24
NOISE64_E_TAIL_REL = 16 * 2.0**-53
