"""Pin the oracle's logits y = H W^T (FlashSampling, Stage 1 step (1)).

bf16 values are dyadic rationals, so the exact dot product is computable with
Python fractions; the oracle's float64 sum must agree to float64 rounding.  A
second check uses numpy's float64 matmul, an independent implementation.
"""
from fractions import Fraction

import numpy as np
import torch

import oracle


def _bf16(shape, std, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


def test_logits_exact_rational():
    H = _bf16((3, 40), 1.0, 1)
    W = _bf16((17, 40), 0.5, 2)
    Y = oracle.logits(H, W)
    Hf = [[Fraction(float(v)) for v in row] for row in H.float().tolist()]
    Wf = [[Fraction(float(v)) for v in row] for row in W.float().tolist()]
    for b in range(3):
        for i in range(17):
            exact = sum(h * w for h, w in zip(Hf[b], Wf[i]))
            assert abs(Y[b, i] - float(exact)) <= 1e-14 * (1 + abs(float(exact)))
    # transposed operands would give [17,3] or wrong values
    assert Y.shape == (3, 17)


def test_logits_match_numpy_float64():
    H = _bf16((5, 512), 1.0, 3)
    W = _bf16((300, 512), 0.02, 4)
    Y = oracle.logits(H, W)
    ref = H.double().numpy() @ W.double().numpy().T
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-13)


def test_logits_ragged_and_extremes():
    # max-magnitude bf16, negative zero and tiny values in one row
    H = torch.tensor([[3.3895e38, -0.0, 1e-30, 1.0]], dtype=torch.bfloat16)
    W = torch.tensor([[0.0, 5.0, 1e-8, 2.0], [1e-38, 1.0, 0.0, -1.0]], dtype=torch.bfloat16)
    Y = oracle.logits(H, W)
    ref = H.double().numpy() @ W.double().numpy().T
    np.testing.assert_allclose(Y, ref, rtol=1e-15)
