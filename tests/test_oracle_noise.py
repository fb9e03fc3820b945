"""Pin the oracle's uniform -> exponential -> Gumbel transforms.

E = -log u and g = -log E are checked against 60-digit decimal arithmetic at the
ends of both midpoint grids and at random grid points, and the ranges they span
are checked against the values the Megatron-LM "fp64 sampling noise" page prints
(noise in [1.1e-16, 36.7], tail widened from about 20 to about 40 nats, smallest
float32 E about 6e-8).
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest
from scipy import stats

import oracle
from conftest import read_golden

getcontext().prec = 60


def _exact(k, bits):
    """(E, g) of u = (k + 1/2) / 2^bits in 60-digit arithmetic."""
    u = (Decimal(2 * k + 1)) / (Decimal(2) ** (bits + 1))
    E = -u.ln()
    g = -E.ln()
    return E, g


def _rel(a, b):
    b = float(b)
    return abs(a - b) / abs(b) if b != 0 else abs(a)


@pytest.mark.parametrize("bits", [23, 52])
def test_transforms_match_decimal(bits):
    rng = np.random.default_rng(11)
    ks = [0, 1, 2, 3, 2**bits // 2 - 1, 2**bits // 2, 2**bits // 2 + 1, 2**bits - 2, 2**bits - 1]
    ks += [int(x) for x in rng.integers(0, 2**bits, size=300, dtype=np.uint64)]
    for k in ks:
        u = (k + 0.5) / 2**bits
        E, g = oracle.noise_of_uniform(u)
        Ex, gx = _exact(k, bits)
        assert _rel(E, Ex) < 4e-16, (k, E, Ex)
        # g crosses zero at E = 1, so bound its error absolutely there
        assert abs(g - float(gx)) < 4e-16 * max(1.0, abs(float(gx))), (k, g, gx)


def _facts():
    return {k: float(v) for k, v in read_golden("megatron_noise_facts.txt")}


def test_noise_range_matches_page():
    f = _facts()
    E_min, g_max = oracle.noise_of_uniform(1 - 0.5 / 2**52)
    E_max, g_min = oracle.noise_of_uniform(0.5 / 2**52)
    # "[1.1e-16, 36.7]" as printed, to the digits printed
    assert round(E_min, 17) == pytest.approx(f["fp64_E_min"], rel=0.01)
    assert round(E_max, 1) == f["fp64_E_max"]
    E32_min, g32_max = oracle.noise_of_uniform(1 - 0.5 / 2**23)
    E32_max, g32_min = oracle.noise_of_uniform(0.5 / 2**23)
    assert E32_min == pytest.approx(f["fp32_E_min"], rel=0.01)       # "about 6e-8"
    # representable tail: ln(E_max / E_min); "about 20" -> "about 40" nats
    span32 = np.log(E32_max / E32_min)
    span64 = np.log(E_max / E_min)
    assert abs(span32 - f["fp32_tail_nats"]) < 1.0
    assert abs(span64 - f["fp64_tail_nats"]) < 1.0
    assert g_max == pytest.approx(-np.log(E_min)) and g_min < 0


@pytest.mark.parametrize("fp64", [False, True])
def test_uniforms_on_grid_and_uniform(fp64):
    bits = 52 if fp64 else 23
    us = np.array([oracle.noise_at(99, 5, 2, i, fp64)[0] for i in range(20000)])
    k = us * 2.0**bits - 0.5
    assert np.all(k == np.floor(k)) and k.min() >= 0 and k.max() < 2**bits
    assert stats.kstest(us, "uniform").pvalue > 1e-4
    # E is standard exponential, g standard Gumbel
    Es = np.array([oracle.noise_at(99, 5, 2, i, fp64)[1] for i in range(20000)])
    assert stats.kstest(Es, "expon").pvalue > 1e-4
    gs = -np.log(Es)
    assert stats.kstest(gs, "gumbel_r").pvalue > 1e-4


def test_offset_and_row_change_the_stream():
    a = [oracle.noise_at(1, 0, 0, i, False)[0] for i in range(64)]
    b = [oracle.noise_at(1, 1, 0, i, False)[0] for i in range(64)]
    c = [oracle.noise_at(1, 0, 1, i, False)[0] for i in range(64)]
    d = [oracle.noise_at(2, 0, 0, i, False)[0] for i in range(64)]
    assert a != b and a != c and a != d
    assert a == [oracle.noise_at(1, 0, 0, i, False)[0] for i in range(64)]


@pytest.mark.parametrize("fp64", [False, True])
def test_noise_row_is_the_per_index_noise(fp64):
    # the whole-row export (used to price residual draws in the verification
    # tests) is the per-index noise of the same row, index by index
    V = 1031
    g = oracle.noise_row(77, 12, 5, V, fp64)
    ref = np.array([oracle.noise_at(77, 12, 5, i, fp64)[2] for i in range(V)])
    assert np.array_equal(g, ref)
