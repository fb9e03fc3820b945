"""Helpers shared by the GPU parity tests (imported by test modules, not collected)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

# Index parity rule: the sampled index must equal the oracle's on every row whose
# oracle top-2 perturbed-score gap exceeds this; closer rows may differ because the
# GPU forms logits in fp32 (and float32 noise in fp32), and are only counted.
GAP = 1e-3
# Logit agreement for bf16 inputs with fp32 accumulation.
LOGIT_TOL = 2e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*args):
    """Print a progress line at once (names the case before a GPU step)."""
    print(*args, flush=True)
    sys.stdout.flush()


def check_index_parity(got, ref_idx, ref_gap, what=""):
    """Assert the parity rule; return the number of near-tie rows (gap <= GAP)."""
    got = np.asarray(got)
    ref_idx = np.asarray(ref_idx)
    ref_gap = np.asarray(ref_gap)
    empty = ref_idx == -1
    assert np.array_equal(got[empty], ref_idx[empty]), f"{what}: rows without a token differ"
    decided = ~empty & (ref_gap > GAP)
    bad = np.nonzero(decided & (got != ref_idx))[0]
    assert bad.size == 0, (f"{what}: {bad.size} decided rows differ, e.g. row {bad[:5]}: "
                           f"got {got[bad[:5]]} oracle {ref_idx[bad[:5]]} gap {ref_gap[bad[:5]]}")
    near = int((~empty & ~decided).sum())
    near_diff = int((~empty & ~decided & (got != ref_idx)).sum())
    say(f"  parity {what}: {decided.sum()} decided rows equal; {near} near-tie rows, "
        f"{near_diff} of them differ")
    return near


def to_dev(*ts, dev):
    return [None if t is None else t.to(dev) for t in ts]
