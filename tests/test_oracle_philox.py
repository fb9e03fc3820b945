"""Pin the oracle's Philox4x32-10 to an independent engine.

The known-answer source is PyTorch's header-only engine
(ATen/core/PhiloxRNGEngine.h), compiled here into a tiny shim.  It is an
independent implementation of the same SC'11 bijection, so a wrong multiplier,
a swapped output word or a missing key bump in the oracle fails these tests.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def torch_philox(tmp_path_factory):
    torch = pytest.importorskip("torch")
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    hdr = os.path.join(inc, "ATen", "core", "PhiloxRNGEngine.h")
    if not os.path.exists(hdr):
        pytest.skip("PyTorch's Philox header is not installed")
    so = str(tmp_path_factory.mktemp("philox") / "torch_philox_shim.so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-I", inc, "-o", so,
                    os.path.join(HERE, "philox_ref", "torch_philox_shim.cpp")], check=True)
    lib = ctypes.CDLL(so)
    lib.torch_philox_block.restype = None
    lib.torch_philox_block.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_void_p]

    def block(ctr, key):
        c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
        out = np.zeros(4, dtype=np.uint32)
        lib.torch_philox_block(c.ctypes.data_as(ctypes.c_void_p), int(key[0]), int(key[1]),
                               out.ctypes.data_as(ctypes.c_void_p))
        return out

    return block


EDGE = [0, 1, 2, 3, 0x7FFFFFFF, 0x80000000, 0xFFFFFFFE, 0xFFFFFFFF, 0x9E3779B9, 1234]


def test_philox_block_matches_independent_engine(torch_philox):
    rng = np.random.default_rng(7)
    cases = [([a, b, c, d], [k0, k1])
             for a, b, c, d, k0, k1 in rng.integers(0, 2**32, size=(400, 6), dtype=np.uint64)]
    for e in EDGE:
        for f in EDGE[::3]:
            cases.append(([e, f, e ^ 0xFFFFFFFF, f], [f, e]))
    cases.append(([0, 0, 0, 0], [0, 0]))
    for ctr, key in cases:
        ctr = [int(x) for x in ctr]
        key = [int(x) for x in key]
        np.testing.assert_array_equal(oracle.philox_block(ctr, key), torch_philox(ctr, key),
                                      err_msg=f"ctr={ctr} key={key}")


def test_philox_words_keying(torch_philox):
    """Counter (j, row, offset lo, offset hi) under key (seed lo, seed hi)."""
    seed = 0x0123456789ABCDEF
    offset = 0xFEDCBA9876543210
    row_ids = np.array([5, 0, 77, 2**32 - 1], dtype=np.uint32)
    words = oracle.philox_words(seed, offset, row_ids, 4, 9)
    for b, r in enumerate(row_ids):
        for j in range(9):
            ref = torch_philox([j, int(r), offset & 0xFFFFFFFF, offset >> 32],
                               [seed & 0xFFFFFFFF, seed >> 32])
            np.testing.assert_array_equal(words[b, j], ref)
    # default row ids are the batch positions
    np.testing.assert_array_equal(oracle.philox_words(seed, offset, None, 3, 2),
                                  oracle.philox_words(seed, offset, [0, 1, 2], 3, 2))


def test_uniform_uses_the_keyed_words(torch_philox):
    """u of vocabulary index i comes from the words of counter i>>2 (fp32 noise,
    word i&3, top 23 bits) or i>>1 (fp64 noise, words 2(i&1) and 2(i&1)+1, top 52
    bits of their concatenation); the words come from the independent engine."""
    seed, offset, r = 1234, 77, 3
    for i in list(range(16)) + [151935, 131071, 2**31 - 1]:
        u, _, _ = oracle.noise_at(seed, offset, r, i, False)
        x = torch_philox([i >> 2, r, offset, 0], [seed, 0])
        k = int(x[i & 3]) >> 9
        assert u == (k + 0.5) / 2**23
        u, _, _ = oracle.noise_at(seed, offset, r, i, True)
        x = torch_philox([i >> 1, r, offset, 0], [seed, 0])
        k = ((int(x[2 * (i & 1)]) << 32) | int(x[2 * (i & 1) + 1])) >> 12
        assert u == (k + 0.5) / 2**52
