"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the sampling method: it only draws the
tensors the method consumes, with the shapes and distributions of the LM-head
workloads on the FlashSampling page (D = 4096, V = 151936 Qwen3-8B-shaped head;
D = 4096, V = 128256 Llama-3-shaped head; D = 8192 wide head) and of the
Megatron-LM tail-rate and chi-square tests.  Every draw uses a CPU
``torch.Generator`` with a fixed seed, so the oracle and the GPU path see
identical bits.  Seeds: W = 0, H = 1, temperatures = 2, bias/mask = 3,
chi-square row = 4, materialised logits and filter settings = 5, speculative
verification inputs = 6.  Reading of
"N(0, s)": s is the standard deviation.
"""
from __future__ import annotations

import math

import numpy as np
import torch

SEED_W, SEED_H, SEED_T, SEED_BIAS, SEED_CHI2, SEED_LOGITS, SEED_SPEC = 0, 1, 2, 3, 4, 5, 6


def _gen(seed: int) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(int(seed))


def weight(V: int, D: int, std: float, seed: int = SEED_W, chunk_rows: int = 8192) -> torch.Tensor:
    """W[V, D] bf16 ~ N(0, std^2), drawn in row chunks so large heads fit in host memory."""
    W = torch.empty((V, D), dtype=torch.bfloat16)
    g = _gen(seed)
    for r0 in range(0, V, chunk_rows):
        r1 = min(V, r0 + chunk_rows)
        W[r0:r1] = (torch.randn((r1 - r0, D), generator=g) * std).to(torch.bfloat16)
    return W


def weight_fp8(V: int, D: int, std: float, seed: int = SEED_W, chunk_rows: int = 8192):
    """An FP8 LM-head weight: (W8 uint8 [V, D] OCP E4M3 bit patterns, scale fp32 [V]).

    Each row of a N(0, std^2) draw is stored as e4m3 values times one float32
    scale, the row's largest magnitude over 448 (the largest E4M3 value), the
    usual per-channel weight quantisation; torch's float8_e4m3fn conversion
    rounds each value to nearest."""
    W8 = torch.empty((V, D), dtype=torch.uint8)
    scale = torch.empty((V,), dtype=torch.float32)
    g = _gen(seed)
    for r0 in range(0, V, chunk_rows):
        r1 = min(V, r0 + chunk_rows)
        w = torch.randn((r1 - r0, D), generator=g) * std
        s = (w.abs().amax(dim=1) / 448.0).clamp_min(1e-30)
        W8[r0:r1] = (w / s[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
        scale[r0:r1] = s
    return W8, scale


_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E2M1_MID = ((_E2M1[1:] + _E2M1[:-1]) / 2).astype(np.float32)


def weight_mxfp4(V: int, D: int, std: float, seed: int = SEED_W, chunk_rows: int = 4096):
    """An MXFP4 LM-head weight: (W4 uint8 [V, D/2], S uint8 [V, D/32]).

    Each block of 32 values of a N(0, std^2) draw (the same draws as weight())
    shares the E8M0 scale 2^X with X = floor(log2(max |w|)) - 2 (2 is the
    largest E2M1 exponent), and each value is rounded to the nearest E2M1 value
    of w / 2^X (ties to the even code, magnitudes above 6 saturate).  Element
    2j sits in the low nibble of byte j, element 2j + 1 in the high nibble."""
    assert D % 32 == 0
    W4 = np.empty((V, D // 2), dtype=np.uint8)
    S = np.empty((V, D // 32), dtype=np.uint8)
    g = _gen(seed)
    for r0 in range(0, V, chunk_rows):
        r1 = min(V, r0 + chunk_rows)
        w = (torch.randn((r1 - r0, D), generator=g) * std).numpy()      # float32
        blk = w.reshape(r1 - r0, D // 32, 32)
        amax = np.abs(blk).max(axis=2).astype(np.float64)
        X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
        X = np.clip(X, -127, 127).astype(np.int64)
        x = blk * np.ldexp(np.float32(1.0), -X).astype(np.float32)[..., None]   # exact
        mag = np.abs(x).reshape(-1)
        # nearest E2M1 magnitude: count the midpoints at or below; on a tie
        # (exactly a midpoint) take the even code
        code = np.searchsorted(_E2M1_MID, mag, side="right")
        tie = (code > 0) & (mag == _E2M1_MID[np.maximum(code - 1, 0)])
        code = np.where(tie & (code % 2 == 1), code - 1, code).astype(np.uint8)
        code |= (np.signbit(x.reshape(-1)) & (code > 0)).astype(np.uint8) << 3
        code = code.reshape(r1 - r0, D)
        W4[r0:r1] = code[:, 0::2] | (code[:, 1::2] << 4)
        S[r0:r1] = (X + 127).astype(np.uint8)
    return torch.from_numpy(W4), torch.from_numpy(S)


def hidden(B: int, D: int, std: float = 1.0, seed: int = SEED_H) -> torch.Tensor:
    """H[B, D] bf16 ~ N(0, std^2)."""
    return (torch.randn((B, D), generator=_gen(seed)) * std).to(torch.bfloat16)


def temperatures(B: int, lo: float = 0.5, hi: float = 1.2, seed: int = SEED_T) -> torch.Tensor:
    """temp[B] fp32 ~ U[lo, hi]."""
    return (torch.rand((B,), generator=_gen(seed), dtype=torch.float64) * (hi - lo) + lo).float()


def bias_with_mask(B: int, V: int, p_mask: float = 0.1, seed: int = SEED_BIAS) -> torch.Tensor:
    """bias[B, V] fp32: N(0, 1) values with Bernoulli(p_mask) entries set to -inf."""
    g = _gen(seed)
    out = torch.empty((B, V), dtype=torch.float32)
    for b in range(B):
        vals = torch.randn((V,), generator=g)
        mask = torch.rand((V,), generator=g) < p_mask
        vals[mask] = float("-inf")
        out[b] = vals
    return out


def chi2_row(n: int = 16, std: float = 2.0, seed: int = SEED_CHI2) -> torch.Tensor:
    """A row of n logits ~ N(0, std^2), fp32."""
    return (torch.randn((n,), generator=_gen(seed)) * std).float()


def tail_depth(r: float) -> float:
    """D = fl32(-ln r): the depth of the tail tokens, rounded to float32."""
    return float(np.float32(-math.log(r)))


def tail_row(V: int, r: float) -> torch.Tensor:
    """The row [0, -D, ..., -D] of V float32 logits with D = fl32(-ln r)."""
    row = torch.full((V,), -tail_depth(r), dtype=torch.float32)
    row[0] = 0.0
    return row


def row_ids(B: int, start: int = 0) -> torch.Tensor:
    """Logical row ids start..start+B-1 as int32 (bit pattern of uint32)."""
    return torch.arange(start, start + B, dtype=torch.int64).to(torch.int32)


def logits(B: int, V: int, std: float = 3.0, seed: int = SEED_LOGITS) -> torch.Tensor:
    """Materialised logits [B, V] float32 ~ N(0, std^2) (the standalone samplers'
    input; std = 3 gives LM-like rows whose top-p sets hold from a few to a few
    thousand tokens)."""
    return (torch.randn((B, V), generator=_gen(seed)) * std).float()


def filter_settings(B: int, V: int, seed: int = SEED_LOGITS + 100):
    """Per-row filter parameters (top_k int32, top_p float32, min_p float32),
    each row drawing which filters are on: top_k in [1, 200] or off (0), top_p
    in [0.5, 0.99] or off (1), min_p in [0.01, 0.3] or off (0)."""
    g = _gen(seed)
    on = torch.rand((3, B), generator=g) < 0.6
    k = torch.randint(1, min(200, V) + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    p = 0.5 + 0.49 * torch.rand((B,), generator=g)
    m = 0.01 + 0.29 * torch.rand((B,), generator=g)
    k = torch.where(on[0], k, torch.zeros_like(k))
    p = torch.where(on[1], p, torch.ones_like(p)).float()
    m = torch.where(on[2], m, torch.zeros_like(m)).float()
    return k, p, m


def spec_decode(B: int, K: int, V: int, std: float = 3.0, draft_noise: float = 1.0,
                temp: float = 0.8, seed: int = SEED_SPEC):
    """Inputs of speculative verification: target logits [B, K+1, V] ~ N(0, std^2),
    draft logits [B, K, V] = the target's first K rows + N(0, draft_noise^2) (a draft
    model that mostly agrees with the target), and draft tokens [B, K] int64 drawn
    from the draft's own softmax at temperature `temp` (torch.multinomial), as a draft
    model's sampler would propose them."""
    g = _gen(seed)
    target = (torch.randn((B, K + 1, V), generator=g) * std).float()
    draft = (target[:, :K] + torch.randn((B, K, V), generator=g) * draft_noise).float().contiguous()
    if K == 0 or B == 0:
        return target, draft, torch.zeros((B, K), dtype=torch.int64)
    probs = torch.softmax(draft.double().reshape(B * K, V) / temp, dim=-1)
    tokens = torch.multinomial(probs, 1, generator=g).reshape(B, K)
    return target, draft, tokens.to(torch.int64).contiguous()
