"""GPU parity of the FP8-weight path (OCP E4M3 weights, one float32 scale per
vocabulary row) against the oracle, through the C ABI.

* The widening of every non-NaN E4M3 code to bf16 is exact: one-hot hidden
  rows pick single weights out of the contraction, which must equal the
  oracle's decode bit for bit (with unit and power-of-two scales).
* NaN codes poison exactly their own row's logits and are never sampled.
* Logits within 2e-3 of the oracle's float64 logits; sampled indices equal
  the oracle's on every row whose top-2 perturbed-score gap exceeds 1e-3, for
  every batch width of a tile, with and without a bias, ragged V, D % 64 != 0,
  several passes per wave, float32 and float64 noise.
* With float64 noise the fused draw equals the standalone sampler's over the
  FP8 path's own float32 logits, bit for bit.
* Full size: the Qwen3-8B-shaped head (D = 4096, V = 151936) quantised per row,
  B in {1, 8, 32, 64}, oracle on sampled rows.
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


def _code_matrix(V, D, seed):
    """W8 [V, D] whose every row holds all 254 non-NaN codes (rotated per row)."""
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes != 0x7F) & (codes != 0xFF)]
    W8 = np.full((V, D), 0x38, dtype=np.uint8)          # 1.0 past the 254 codes
    for i in range(V):
        W8[i, :codes.size] = np.roll(codes, 17 * i + seed)
    return W8


@pytest.mark.parametrize("scale_kind", ["unit", "pow2"])
def test_w8_decode_every_code_exact(dev, scale_kind):
    V, D = 16, 256
    say(f"fp8 decode of every code, scale={scale_kind}")
    W8 = _code_matrix(V, D, seed=3)
    if scale_kind == "unit":
        scale = np.ones(V, dtype=np.float32)
    else:
        scale = np.ldexp(np.ones(V), np.arange(V) - 10).astype(np.float32)
    H = torch.eye(D, dtype=torch.float32).to(torch.bfloat16)     # B = D one-hot rows
    Y = fs.debug_logits_w8(H.to(dev), torch.from_numpy(W8).to(dev), torch.from_numpy(scale).to(dev))
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    ref = (oracle.e4m3_to_double(W8) * scale.astype(np.float64)[:, None]).T   # [D, V]
    assert np.isfinite(Y).all()
    np.testing.assert_array_equal(Y, ref.astype(np.float32))
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)   # exact in fp32


@pytest.mark.parametrize("fp64", [False, True])
def test_w8_nan_rows_never_sampled(dev, fp64):
    B, D, V = 8, 64, 500
    say(f"fp8 NaN codes fp64={fp64}")
    W8, scale = synthetic.weight_fp8(V, D, std=0.5, seed=5)
    W8 = W8.numpy().copy()
    nan_rows = [0, 3, 77, 499]
    for k, r in enumerate(nan_rows):
        W8[r, (13 * k) % D] = 0x7F if k % 2 == 0 else 0xFF
    H = synthetic.hidden(B, D, seed=6)
    temp = synthetic.temperatures(B, seed=7)
    temp[2] = 0.0
    Hd, td = to_dev(H, temp, dev=dev)
    W8d, sd = torch.from_numpy(W8).to(dev), scale.to(dev)
    Y = fs.debug_logits_w8(Hd, W8d, sd).cpu().numpy()
    assert np.isnan(Y[:, nan_rows]).all()
    others = np.setdiff1d(np.arange(V), nan_rows)
    assert np.isfinite(Y[:, others]).all()
    got = fs.sample_fused_w8(Hd, W8d, sd, td, seed=11, offset=2, fp64_noise=fp64).cpu().numpy()
    assert not np.isin(got, nan_rows).any()
    ref, gap, _ = oracle.sample_fused_w8(H, W8, scale.numpy(), temp.numpy(), seed=11, offset=2,
                                         fp64_noise=fp64)
    check_index_parity(got, ref, gap, "fp8 NaN rows")


LOGIT_SHAPES = [
    (4, 512, 32768),
    (37, 208, 1001),      # ragged B, D % 64 != 0, V % 16 != 0
    (70, 528, 777),       # two batch tiles
    (1, 16, 5),           # the smallest D
    (16, 4096, 2000),
    (33, 64, 4099),
]


@pytest.mark.parametrize("B,D,V", LOGIT_SHAPES)
def test_w8_logits_match_oracle(dev, B, D, V):
    say(f"fp8 debug logits B={B} D={D} V={V}")
    H = synthetic.hidden(B, D, seed=11)
    W8, scale = synthetic.weight_fp8(V, D, std=0.02 if D >= 512 else 0.3, seed=12)
    Hd, W8d, sd = to_dev(H, W8, scale, dev=dev)
    Y = fs.debug_logits_w8(Hd, W8d, sd)
    torch.cuda.synchronize()
    ref = oracle.logits_w8(H, W8.numpy(), scale.numpy())
    err = np.abs(Y.cpu().double().numpy() - ref).max()
    say(f"  max |dy| = {err:.3e}")
    assert err <= LOGIT_TOL


def _case(B, D, V, *, bias=False, greedy_rows=(), seed_base=0, w_std=0.02):
    H = synthetic.hidden(B, D, seed=120 + seed_base)
    W8, scale = synthetic.weight_fp8(V, D, std=w_std, seed=121 + seed_base)
    temp = synthetic.temperatures(B, seed=122 + seed_base)
    for r in greedy_rows:
        temp[r] = [0.0, -1.0, float("nan")][r % 3]
    bb = synthetic.bias_with_mask(B, V, 0.1, seed=123 + seed_base) if bias else None
    return H, W8, scale, temp, bb


FP8_CASES = [
    dict(B=4, D=512, V=32768),
    dict(B=37, D=208, V=1001, bias=True, greedy_rows=(0, 5, 9)),
    dict(B=70, D=528, V=777, bias=True),
    dict(B=16, D=4096, V=5000, greedy_rows=(3,)),
    dict(B=3, D=16, V=13, w_std=1.0),
    dict(B=24, D=96, V=1500, bias=True),
    dict(B=48, D=128, V=2500, greedy_rows=(1,)),
    dict(B=64, D=272, V=3001),
    dict(B=64, D=64, V=170001, greedy_rows=(2, 40)),
    dict(B=20, D=64, V=170001, bias=True),
]


@pytest.mark.parametrize("fp64", [False, True])
@pytest.mark.parametrize("case", FP8_CASES)
def test_w8_sampling_parity(dev, case, fp64):
    case = dict(case)
    B, D, V = case.pop("B"), case.pop("D"), case.pop("V")
    say(f"fp8 fused sample B={B} D={D} V={V} fp64={fp64} {case}")
    H, W8, scale, temp, bias = _case(B, D, V, **case)
    Hd, W8d, sd, td, bd = to_dev(H, W8, scale, temp, bias, dev=dev)
    got = fs.sample_fused_w8(Hd, W8d, sd, td, bd, seed=1234, offset=5, fp64_noise=fp64)
    torch.cuda.synchronize()
    ref, gap, _ = oracle.sample_fused_w8(H, W8.numpy(), scale.numpy(), temp.numpy(),
                                         None if bias is None else bias.numpy(), seed=1234,
                                         offset=5, fp64_noise=fp64)
    check_index_parity(got.cpu().numpy(), ref, gap, f"fp8 B={B} V={V} fp64={fp64}")


@pytest.mark.parametrize("B", [16, 20, 40])
def test_w8_degenerate_scales(dev, B):
    """Rows whose scale is zero (an all-zero row quantises so), negative or NaN,
    at batch widths whose kernels fold the noise into the sums (16, 48 columns)
    and one that adds it after the k-loop (32): the logit is the product of
    the scale and the sum either way."""
    D, V = 512, 3000
    say(f"fp8 degenerate scales B={B}")
    H, W8, scale, temp, bias = _case(B, D, V, bias=True, greedy_rows=(1,), seed_base=70)
    scale = scale.clone()
    scale[[5, 6, 77, 1500]] = 0.0
    scale[[9, 2999]] = -scale[[9, 2999]]
    scale[300] = float("nan")
    # zero-scale tokens carry logit 0: with a large bias they must win
    bias[0, [5, 6, 77, 1500]] = 100.0
    bias[2, 77] = 200.0
    Hd, W8d, sd, td, bd = to_dev(H, W8, scale, temp, bias, dev=dev)
    got = fs.sample_fused_w8(Hd, W8d, sd, td, bd, seed=41, offset=42)
    torch.cuda.synchronize()
    ref, gap, _ = oracle.sample_fused_w8(H, W8.numpy(), scale.numpy(), temp.numpy(), bias.numpy(),
                                         seed=41, offset=42)
    got = got.cpu().numpy()
    check_index_parity(got, ref, gap, f"fp8 degenerate scales B={B}")
    assert got[0] in (5, 6, 77, 1500) and got[2] == 77


def test_w8_fused_equals_standalone_on_its_logits(dev):
    say("fp8 fused vs standalone on the FP8 path's logits")
    B, D, V = 40, 512, 4096
    H, W8, scale, temp, _ = _case(B, D, V, seed_base=30)
    Hd, W8d, sd, td = to_dev(H, W8, scale, temp, dev=dev)
    rid = torch.arange(100, 100 + B, dtype=torch.int32, device=dev)
    y = fs.debug_logits_w8(Hd, W8d, sd)
    a = fs.sample_fused_w8(Hd, W8d, sd, td, seed=5, offset=6, row_ids=rid, fp64_noise=True)
    b = fs.sample_logits(y, td, seed=5, offset=6, row_ids=rid, fp64_noise=True)
    assert torch.equal(a, b)
    a = fs.sample_fused_w8(Hd, W8d, sd, td, seed=5, offset=6, row_ids=rid).cpu().numpy()
    ref, gap, _ = oracle.sample_logits(y.cpu().numpy(), temp.numpy(), seed=5, offset=6,
                                       row_ids=np.arange(100, 100 + B, dtype=np.uint32))
    check_index_parity(a, ref, gap, "fp8 fused vs oracle on its logits")


def test_w8_replay_and_permutation(dev):
    say("fp8 replay and batch permutation")
    B, D, V = 33, 256, 3001
    H, W8, scale, temp, bias = _case(B, D, V, bias=True, seed_base=40)
    Hd, W8d, sd, td, bd = to_dev(H, W8, scale, temp, bias, dev=dev)
    rid = torch.arange(B, dtype=torch.int32, device=dev)
    a = fs.sample_fused_w8(Hd, W8d, sd, td, bd, seed=3, offset=9, row_ids=rid).clone()
    assert torch.equal(a, fs.sample_fused_w8(Hd, W8d, sd, td, bd, seed=3, offset=9, row_ids=rid))
    perm = torch.randperm(B, generator=torch.Generator().manual_seed(4)).to(dev)
    p = fs.sample_fused_w8(Hd[perm].contiguous(), W8d, sd, td[perm].contiguous(),
                           bd[perm].contiguous(), seed=3, offset=9, row_ids=rid[perm].contiguous())
    assert torch.equal(p, a[perm])


def test_w8_float8_dtype_and_errors(dev):
    B, D, V = 2, 32, 100
    H, W8, scale, temp, _ = _case(B, D, V, seed_base=50)
    Hd, W8d, sd, td = to_dev(H, W8, scale, temp, dev=dev)
    a = fs.sample_fused_w8(Hd, W8d, sd, td, seed=1, offset=1)
    b = fs.sample_fused_w8(Hd, W8d.view(torch.float8_e4m3fn), sd, td, seed=1, offset=1)
    assert torch.equal(a, b)
    lib = fs.load_library()
    out = torch.empty(B, dtype=torch.int64, device=dev)
    ws = torch.zeros(lib.fs_workspace_bytes(B, V, 0), dtype=torch.uint8, device=dev)
    args = lambda Dx, scale_ptr: (fs._ptr(Hd), fs._ptr(W8d), scale_ptr, B, Dx, V, fs._ptr(td), None,
                                  1, 1, fs._ptr(out), None, 0, fs._ptr(ws), ws.numel(),
                                  fs._stream(dev))
    assert lib.fs_sample_fused_w8(*args(24, fs._ptr(sd))) == 2       # D % 16 != 0
    assert lib.fs_sample_fused_w8(*args(D, None)) == 1               # no scales
    assert lib.fs_sample_fused_w8(*args(D, fs._ptr(sd))) == 0


@pytest.fixture(scope="module")
def qwen_head_fp8(dev):
    say("generating the FP8 D=4096 V=151936 head")
    W8, scale = synthetic.weight_fp8(151936, 4096, std=0.02)
    H = synthetic.hidden(64, 4096)
    temp = synthetic.temperatures(64)
    return H, W8, scale, temp, W8.to(dev), scale.to(dev)


def test_w8_qwen_head_sampled_rows(dev, qwen_head_fp8):
    H, W8, scale, temp, W8d, sd = qwen_head_fp8
    rows = np.array([0, 1, 7, 8, 31, 32, 63])
    say(f"oracle rows {rows.tolist()} of the FP8 D=4096 V=151936 head")
    ref, gap, _ = oracle.sample_fused_w8(H[rows], W8.numpy(), scale.numpy(), temp[rows].numpy(),
                                         seed=1234, offset=17, row_ids=rows.astype(np.uint32))
    for B in (1, 8, 32, 64):
        say(f"fp8 fused B={B}")
        got = fs.sample_fused_w8(H[:B].to(dev), W8d, sd, temp[:B].to(dev), seed=1234, offset=17)
        torch.cuda.synchronize()
        sel = rows < B
        check_index_parity(got.cpu().numpy()[rows[sel]], ref[sel], gap[sel], f"fp8 qwen B={B}")
    Y = fs.debug_logits_w8(H.to(dev), W8d, sd)
    torch.cuda.synchronize()
    for r in (0, 63):
        err = np.abs(Y[r].cpu().double().numpy()
                     - oracle.logits_w8(H[r:r + 1], W8.numpy(), scale.numpy())[0]).max()
        say(f"  row {r}: max |dy| = {err:.3e}")
        assert err <= LOGIT_TOL
