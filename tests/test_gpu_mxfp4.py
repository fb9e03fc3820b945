"""GPU parity of the MXFP4-weight path (E2M1 elements, an E8M0 scale per block
of 32 along D) against the oracle, through the C ABI.

* The on-chip widening is exact: one-hot hidden rows pick single elements out
  of the contraction, which must equal the oracle's decode times the block
  scale bit for bit, for every code in both nibble positions.
* Logits within 2e-3 of the oracle's float64 logits; sampled indices equal
  the oracle's on every row whose top-2 perturbed-score gap exceeds 1e-3, for
  every batch width, with and without a bias, D an odd multiple of 256 (in
  both the 256-k and the 512-k chunk layouts), several passes per wave,
  float32 and float64 noise.
* Float64 noise: the fused draw equals the standalone sampler's over the
  path's own float32 logits, bit for bit.
* Full size: the Qwen3-8B-shaped head (D = 4096, V = 151936) in MXFP4,
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


def _codes(W4):
    W4 = np.asarray(W4, dtype=np.uint8)
    return np.stack([W4 & 15, W4 >> 4], axis=-1).reshape(W4.shape[0], -1)


def test_mxfp4_decode_every_code_exact(dev):
    V, D = 16, 256
    say("mxfp4 decode of every code in both nibbles, block scales 2^-125 to 2^125")
    codes = (np.arange(D)[None, :] + np.arange(V)[:, None]) % 16
    W4 = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    # block scales from both ends of the range the widening keeps exact (every
    # scaled value a normal bf16 number: codes 2 to 252) and around 1
    codes_e = np.array([2, 3, 60, 124, 125, 126, 127, 128, 129, 130, 200, 250, 252])
    S = codes_e[(np.arange(V)[:, None] + np.arange(D // 32)[None, :]) % len(codes_e)].astype(np.uint8)
    H = torch.eye(D, dtype=torch.float32).to(torch.bfloat16)        # B = D one-hot rows
    Y = fs.debug_logits_mxfp4(H.to(dev), torch.from_numpy(W4).to(dev), torch.from_numpy(S).to(dev))
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    vals = oracle.e2m1_to_double(codes.reshape(-1)).reshape(V, D)
    scale = np.repeat(oracle.e8m0_to_double(S.reshape(-1)).reshape(V, D // 32), 32, axis=1)
    ref = (vals * scale).T                                           # [D, V]
    np.testing.assert_array_equal(Y, ref.astype(np.float32))


LOGIT_SHAPES = [
    (4, 512, 32768),
    (37, 256, 1001),
    (70, 768, 777),        # an odd number of 256-k chunks, two batch tiles
    (16, 4096, 2000),
    (1, 256, 5),
    (32, 768, 3000),       # 32 columns in 512-k chunks, the last one half past D
    (3, 4352, 1500),       # scales read per pair (past 4096 k)
    (64, 4352, 700),
]


@pytest.mark.parametrize("B,D,V", LOGIT_SHAPES)
def test_mxfp4_logits_match_oracle(dev, B, D, V):
    say(f"mxfp4 debug logits B={B} D={D} V={V}")
    H = synthetic.hidden(B, D, seed=31)
    W4, S = synthetic.weight_mxfp4(V, D, std=0.02 if D >= 512 else 0.3, seed=32)
    Hd, W4d, Sd = to_dev(H, W4, S, dev=dev)
    Y = fs.debug_logits_mxfp4(Hd, W4d, Sd)
    torch.cuda.synchronize()
    ref = oracle.logits_w4(H, W4.numpy(), S.numpy())
    err = np.abs(Y.cpu().double().numpy() - ref).max()
    say(f"  max |dy| = {err:.3e}")
    assert err <= LOGIT_TOL


def _case(B, D, V, *, bias=False, greedy_rows=(), seed_base=0, w_std=0.02):
    H = synthetic.hidden(B, D, seed=320 + seed_base)
    W4, S = synthetic.weight_mxfp4(V, D, std=w_std, seed=321 + seed_base)
    temp = synthetic.temperatures(B, seed=322 + seed_base)
    for r in greedy_rows:
        temp[r] = [0.0, -1.0, float("nan")][r % 3]
    bb = synthetic.bias_with_mask(B, V, 0.1, seed=323 + seed_base) if bias else None
    return H, W4, S, temp, bb


MXFP4_CASES = [
    dict(B=4, D=512, V=32768),
    dict(B=37, D=256, V=1001, bias=True, greedy_rows=(0, 5, 9)),
    dict(B=70, D=768, V=777, bias=True),
    dict(B=16, D=4096, V=5000, greedy_rows=(3,)),
    dict(B=3, D=256, V=13, w_std=1.0),
    dict(B=24, D=1280, V=1500, bias=True),
    dict(B=48, D=256, V=2500, greedy_rows=(1,)),
    dict(B=64, D=512, V=3001),
    dict(B=64, D=256, V=170001, greedy_rows=(2, 40)),
    dict(B=20, D=256, V=170001, bias=True),
    dict(B=30, D=768, V=4099, greedy_rows=(4,)),    # 512-k chunks, the last one half past D
    dict(B=9, D=1280, V=2048, bias=True),           # 16 columns, bias, 512-k chunks
    # past 4096 k a row's scales no longer fit the LDS row: read per pair
    dict(B=5, D=4352, V=3001, greedy_rows=(2,)),
    dict(B=50, D=4352, V=2001, bias=True),
]


@pytest.mark.parametrize("fp64", [False, True])
@pytest.mark.parametrize("case", MXFP4_CASES)
def test_mxfp4_sampling_parity(dev, case, fp64):
    case = dict(case)
    B, D, V = case.pop("B"), case.pop("D"), case.pop("V")
    say(f"mxfp4 fused sample B={B} D={D} V={V} fp64={fp64} {case}")
    H, W4, S, temp, bias = _case(B, D, V, **case)
    Hd, W4d, Sd, td, bd = to_dev(H, W4, S, temp, bias, dev=dev)
    got = fs.sample_fused_mxfp4(Hd, W4d, Sd, td, bd, seed=1234, offset=5, fp64_noise=fp64)
    torch.cuda.synchronize()
    ref, gap, _ = oracle.sample_fused_w4(H, W4.numpy(), S.numpy(), temp.numpy(),
                                         None if bias is None else bias.numpy(), seed=1234,
                                         offset=5, fp64_noise=fp64)
    check_index_parity(got.cpu().numpy(), ref, gap, f"mxfp4 B={B} V={V} fp64={fp64}")


def test_mxfp4_fused_equals_standalone_on_its_logits(dev):
    say("mxfp4 fused vs standalone on the path's logits")
    B, D, V = 40, 512, 4096
    H, W4, S, temp, _ = _case(B, D, V, seed_base=30)
    Hd, W4d, Sd, td = to_dev(H, W4, S, temp, dev=dev)
    rid = torch.arange(100, 100 + B, dtype=torch.int32, device=dev)
    y = fs.debug_logits_mxfp4(Hd, W4d, Sd)
    a = fs.sample_fused_mxfp4(Hd, W4d, Sd, td, seed=5, offset=6, row_ids=rid, fp64_noise=True)
    b = fs.sample_logits(y, td, seed=5, offset=6, row_ids=rid, fp64_noise=True)
    assert torch.equal(a, b)


def test_mxfp4_argument_errors(dev):
    B, D, V = 2, 256, 100
    H, W4, S, temp, _ = _case(B, D, V, seed_base=50)
    Hd, W4d, Sd, td = to_dev(H, W4, S, temp, dev=dev)
    lib = fs.load_library()
    out = torch.empty(B, dtype=torch.int64, device=dev)
    ws = torch.zeros(lib.fs_workspace_bytes(B, V, 0), dtype=torch.uint8, device=dev)
    args = lambda Dx, sp: (fs._ptr(Hd), fs._ptr(W4d), sp, B, Dx, V, fs._ptr(td), None, 1, 1,
                           fs._ptr(out), None, 0, fs._ptr(ws), ws.numel(), fs._stream(dev))
    assert lib.fs_sample_fused_mxfp4(*args(128, fs._ptr(Sd))) == 2      # D % 256 != 0
    assert lib.fs_sample_fused_mxfp4(*args(D, None)) == 1               # no scales
    assert lib.fs_sample_fused_mxfp4(*args(D, fs._ptr(Sd))) == 0


def test_mxfp4_qwen_head_sampled_rows(dev):
    say("generating the MXFP4 D=4096 V=151936 head")
    W4, S = synthetic.weight_mxfp4(151936, 4096, std=0.02)
    H = synthetic.hidden(64, 4096)
    temp = synthetic.temperatures(64)
    W4d, Sd = W4.to(dev), S.to(dev)
    rows = np.array([0, 1, 7, 8, 31, 32, 63])
    say(f"oracle rows {rows.tolist()} of the MXFP4 head")
    ref, gap, _ = oracle.sample_fused_w4(H[rows], W4.numpy(), S.numpy(), temp[rows].numpy(),
                                         seed=1234, offset=17, row_ids=rows.astype(np.uint32))
    for B in (1, 8, 32, 64):
        say(f"mxfp4 fused B={B}")
        got = fs.sample_fused_mxfp4(H[:B].to(dev), W4d, Sd, temp[:B].to(dev), seed=1234, offset=17)
        torch.cuda.synchronize()
        sel = rows < B
        check_index_parity(got.cpu().numpy()[rows[sel]], ref[sel], gap[sel], f"mxfp4 qwen B={B}")
