"""GPU parity of the repetition penalty (fs_repetition_penalty) and of the
card's whole sample pipeline (penalty, temperature, top-k, top-p, min-p,
draw) against the oracle, through the C ABI.

* The penalised logits equal the oracle's bit for bit (both are the correctly
  rounded float32 product or quotient): duplicates, padding outside [0, V),
  zero and -inf logits, rows whose penalty is 0 or NaN (unchanged), V % 4 != 0
  (scalar loads), several chunks a row, in place and out of place.
* The pipeline's draws equal the oracle's composition (oracle penalty, then
  the oracle's filtered draw) on every row whose filter decisions lie further
  than 2e-5 from their boundaries and whose top-2 kept perturbed-score gap
  exceeds 1e-3.
"""
import numpy as np
import pytest
import torch

import decode_exact_categorical_amd as fs
import oracle
import synthetic
from gpu_common import GAP, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _inputs(B, V, L, seed):
    x = synthetic.logits(B, V, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    prev = torch.randint(0, V, (B, L), generator=g, dtype=torch.int64)
    if L >= 4:
        prev[:, 1] = prev[:, 0]                      # a duplicate
        prev[:, 2] = -1                              # padding
        prev[:, 3] = V
    x[0, :3] = 0.0
    if L >= 3:
        prev[0, :3] = torch.arange(3)
    if L >= 1:
        x[min(1, B - 1), int(prev[min(1, B - 1), 0])] = -float("inf")
    pen = (0.5 + 1.5 * torch.rand(B, generator=g)).float()
    if B >= 4:
        pen[2], pen[3] = 0.0, float("nan")           # rows left unchanged
    return x, prev, pen


@pytest.mark.parametrize("B,V,L", [(8, 128256, 64), (5, 5003, 300), (3, 100, 4), (16, 20000, 1),
                                   (2, 9000, 0)])
def test_penalty_bit_exact(dev, B, V, L):
    say(f"repetition penalty B={B} V={V} L={L}")
    x, prev, pen = _inputs(B, V, L, seed=60 + V)
    ref = oracle.repetition_penalty(x.numpy(), prev.numpy(), pen.numpy())
    xd, pd, qd = x.to(dev), prev.to(dev), pen.to(dev)
    got = fs.repetition_penalty(xd, pd, qd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), ref)
    fs.repetition_penalty(xd, pd, qd, out=xd)        # in place
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xd.cpu().numpy(), ref)


def test_sample_pipeline(dev):
    B, V, L = 24, 50000, 128
    say("penalty + temperature + top-k + top-p + draw")
    x, prev, _ = _inputs(B, V, L, seed=70)
    t = synthetic.temperatures(B, seed=71)
    kw = dict(top_k=50, top_p=0.95)
    got = fs.sample(x.to(dev), t.to(dev), repetition_penalty=1.3, prev_tokens=prev.to(dev),
                    seed=21, offset=5, **kw)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    xp = oracle.repetition_penalty(x.numpy(), prev.numpy(), 1.3)
    idx, gap, margin = oracle.sample_logits_filtered(xp, t.numpy(), seed=21, offset=5, **kw)
    decided = (margin > 2e-5) & (gap > GAP)
    assert decided.mean() >= 0.6
    np.testing.assert_array_equal(got[decided], idx[decided])
