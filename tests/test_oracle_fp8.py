"""Pins of the oracle's FP8-weight path (OCP E4M3 weights with one scale per
vocabulary row), independent of the oracle's own code: torch's float8_e4m3fn
conversion for the decode, exact rational arithmetic for the scaled dot
products, and the bf16 path of the oracle itself (every E4M3 value is exactly a
bf16 value, so with unit scales both paths must agree bit for bit)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic


def test_e4m3_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_to_double(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_special_values():
    d = oracle.e4m3_to_double(np.array([0x7E, 0x08, 0x07, 0x01, 0x38, 0x00, 0x80, 0x7F, 0xFF, 0xFE],
                                       dtype=np.uint8))
    assert d[0] == 448.0                    # largest finite value, no infinities
    assert d[1] == 2.0 ** -6                # smallest normal
    assert d[2] == 7 * 2.0 ** -9            # largest subnormal
    assert d[3] == 2.0 ** -9                # smallest subnormal
    assert d[4] == 1.0
    assert d[5] == 0.0 and not np.signbit(d[5])
    assert d[6] == 0.0 and np.signbit(d[6])
    assert np.isnan(d[7]) and np.isnan(d[8])
    assert d[9] == -448.0
    pos = oracle.e4m3_to_double(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)         # codes 0..126 increase strictly


def test_logits_w8_exact_rational():
    rng = np.random.default_rng(3)
    B, D, V = 2, 24, 5
    H = torch.from_numpy(rng.standard_normal((B, D))).to(torch.bfloat16)
    W8 = rng.integers(0, 256, size=(V, D), dtype=np.uint8)
    W8[W8 == 0x7F] = 0x7E
    W8[W8 == 0xFF] = 0xFE
    scale = rng.uniform(0.01, 2.0, size=V).astype(np.float32)
    got = oracle.logits_w8(H, W8, scale)
    dec = torch.from_numpy(W8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    h = H.to(torch.float64).numpy()
    for b in range(B):
        for i in range(V):
            exact = Fraction(float(scale[i])) * sum(Fraction(float(h[b, d])) * Fraction(float(dec[i, d]))
                                                    for d in range(D))
            assert abs(got[b, i] - float(exact)) <= 1e-14 * max(1.0, abs(float(exact)))


@pytest.mark.parametrize("fp64", [False, True])
def test_w8_path_equals_bf16_path_at_unit_scale(fp64):
    B, D, V = 5, 64, 3000
    W8, _ = synthetic.weight_fp8(V, D, std=0.3, seed=9)
    Wbf = W8.view(torch.float8_e4m3fn).to(torch.bfloat16)      # exact: e4m3 is a subset of bf16
    assert torch.equal(Wbf.float(), W8.view(torch.float8_e4m3fn).float())
    H = synthetic.hidden(B, D, seed=10)
    ones = np.ones(V, dtype=np.float32)
    np.testing.assert_array_equal(oracle.logits_w8(H, W8.numpy(), ones), oracle.logits(H, Wbf))
    temp = synthetic.temperatures(B, seed=11).numpy()
    a = oracle.sample_fused_w8(H, W8.numpy(), ones, temp, seed=5, offset=6, fp64_noise=fp64)
    b = oracle.sample_fused(H, Wbf, temp, seed=5, offset=6, fp64_noise=fp64)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_w8_scale_multiplies_each_row():
    B, D, V = 3, 32, 200
    W8, scale = synthetic.weight_fp8(V, D, std=0.02, seed=12)
    H = synthetic.hidden(B, D, seed=13)
    y1 = oracle.logits_w8(H, W8.numpy(), np.ones(V, dtype=np.float32))
    ys = oracle.logits_w8(H, W8.numpy(), scale.numpy())
    np.testing.assert_allclose(ys, y1 * scale.numpy().astype(np.float64)[None, :], rtol=1e-15, atol=0)


def test_weight_fp8_generator_round_trip():
    V, D, std = 64, 256, 0.02
    W8, scale = synthetic.weight_fp8(V, D, std=std, seed=0)
    W = synthetic.weight(V, D, std=std, seed=0).float()   # same generator draws, kept in bf16
    deq = W8.view(torch.float8_e4m3fn).float() * scale[:, None]
    assert np.isfinite(deq.numpy()).all()
    assert (W8.view(torch.float8_e4m3fn).float().abs().amax(dim=1) == 448.0).all()
    rel = ((deq - W).abs() / W.abs().clamp_min(1e-6)).numpy()
    big = W.abs().numpy() > std * 0.5          # away from the subnormal range of each row
    assert np.quantile(rel[big], 0.99) < 2.0 ** -3
