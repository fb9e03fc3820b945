"""Pins of the oracle's MXFP4-weight path (FP4 E2M1 elements in blocks of 32
sharing an E8M0 scale), independent of the oracle's own code: PyTorch's
E2M1 and E8M0 decoders, exact rational arithmetic for the scaled dot products,
and the bf16 path of the oracle (every scaled E2M1 value of a moderate scale
is exactly a bf16 value, so with unit scales both paths agree bit for bit)."""
import sys
import types
import unittest
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic


def _torch_e2m1_decoder():
    """PyTorch's own E2M1 decoder (a testing helper); its module imports a test
    package that is not installed here, which a stand-in satisfies."""
    if "expecttest" not in sys.modules:
        stub = types.ModuleType("expecttest")
        stub.TestCase = unittest.TestCase
        sys.modules["expecttest"] = stub
    from torch.testing._internal.common_quantized import _floatx_unpacked_to_f32
    return lambda codes: _floatx_unpacked_to_f32(torch.as_tensor(codes, dtype=torch.uint8), 2, 1)


def _unpack(W4):
    W4 = np.asarray(W4, dtype=np.uint8)
    return np.stack([W4 & 15, W4 >> 4], axis=-1).reshape(W4.shape[0], -1)


def test_e2m1_decode_every_code_matches_torch():
    try:
        dec = _torch_e2m1_decoder()
    except Exception as e:           # pragma: no cover - depends on the torch build
        pytest.skip(f"torch E2M1 decoder unavailable: {e}")
    codes = np.arange(16, dtype=np.uint8)
    ref = dec(codes).double().numpy()
    got = oracle.e2m1_to_double(codes)
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(ref))


def test_e8m0_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.e8m0_to_double(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_logits_w4_exact_rational():
    rng = np.random.default_rng(7)
    B, D, V = 2, 64, 5
    H = torch.from_numpy(rng.standard_normal((B, D))).to(torch.bfloat16)
    W4 = rng.integers(0, 256, size=(V, D // 2), dtype=np.uint8)
    S = rng.integers(110, 140, size=(V, D // 32), dtype=np.uint8)
    got = oracle.logits_w4(H, W4, S)
    codes = _unpack(W4)
    e2m1 = {c: Fraction(v) for c, v in enumerate(_torch_e2m1_decoder()(np.arange(16)).tolist())}
    h = H.to(torch.float64).numpy()
    for b in range(B):
        for i in range(V):
            exact = sum(Fraction(float(h[b, d])) * e2m1[int(codes[i, d])]
                        * Fraction(2) ** (int(S[i, d // 32]) - 127) for d in range(D))
            assert abs(got[b, i] - float(exact)) <= 1e-14 * max(1.0, abs(float(exact)))


def test_w4_unit_scales_equal_the_bf16_path():
    rng = np.random.default_rng(8)
    B, D, V = 4, 128, 300
    W4 = rng.integers(0, 256, size=(V, D // 2), dtype=np.uint8)
    S = np.full((V, D // 32), 127, dtype=np.uint8)
    vals = _torch_e2m1_decoder()(_unpack(W4).reshape(-1)).reshape(V, D)
    Wbf = vals.to(torch.bfloat16)
    assert torch.equal(Wbf.float(), vals.float())
    H = synthetic.hidden(B, D, seed=9)
    np.testing.assert_array_equal(oracle.logits_w4(H, W4, S), oracle.logits(H, Wbf))


def test_w4_nibble_order_and_block_scales():
    D, V = 64, 3
    W4 = np.zeros((V, D // 2), dtype=np.uint8)
    W4[0, 0] = 0x02 << 4            # element 1 (high nibble of byte 0) = 1.0
    W4[1, 0] = 0x07                 # element 0 (low nibble) = 6.0
    W4[2, 16] = 0x0D                # element 32 (first of block 1) = -3.0
    S = np.full((V, D // 32), 127, dtype=np.uint8)
    S[2, 1] = 130                   # block 1 of row 2 scaled by 8
    H = torch.zeros((1, D))
    H[0, 0], H[0, 1], H[0, 32] = 1.0, 2.0, 0.5
    y = oracle.logits_w4(H.to(torch.bfloat16), W4, S)[0]
    np.testing.assert_array_equal(y, [2.0, 6.0, -3.0 * 8 * 0.5])


def test_weight_mxfp4_generator():
    V, D, std = 32, 256, 0.02
    W4, S = synthetic.weight_mxfp4(V, D, std=std, seed=0)
    W = synthetic.weight(V, D, std=std, seed=0).double().numpy()
    vals = _torch_e2m1_decoder()(_unpack(W4.numpy()).reshape(-1)).double().numpy().reshape(V, D)
    scale = np.repeat(oracle.e8m0_to_double(S.numpy().reshape(-1)).reshape(V, D // 32), 32, axis=1)
    deq = vals * scale
    blk_max = np.repeat(np.abs(W).reshape(V, D // 32, 32).max(axis=2), 32, axis=1)
    # every block's largest magnitude maps into [4, 8) scale units; up to 6
    # units the E2M1 grid steps are 0.5, 1 and 2 units below 2, 4 and 6, and a
    # value is at most half a step off (plus the bf16 rounding of W itself)
    u = np.abs(W) / scale
    assert ((blk_max / scale >= 4 - 1e-6) & (blk_max / scale < 8 + 1e-6)).all()
    half_step = np.where(u < 2, 0.25, np.where(u < 4, 0.5, 1.0))
    ok = u <= 6
    assert (np.abs(deq - W)[ok] <= (half_step * scale)[ok] + 2.0 ** -8 * np.abs(W)[ok]).all()
    assert (np.abs(deq[~ok]) == 6 * scale[~ok]).all()          # saturated
