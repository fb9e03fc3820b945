"""CPU oracle for exact categorical sampling (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library in
``decode_exact_categorical_amd``) never imports it, and the two share no code.

The arithmetic lives in ``fs_oracle.c`` (plain C, float64, OpenMP over the
vocabulary); this module only marshals numpy arrays into it.  What each C
function computes, and which passage of the source pages it follows, is stated
in the header of ``fs_oracle.c``.  Statistical helpers used by the pins
(Poisson intervals, chi-square) live in ``oracle/stats.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fs_oracle.c")
_LIB = os.path.join(_HERE, "libfs_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile fs_oracle.c into libfs_oracle.so (gcc, -O2, OpenMP, strict IEEE)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, u64, u32, i32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int
        lib.oracle_num_threads.restype = i32
        lib.oracle_num_threads.argtypes = []
        lib.oracle_set_num_threads.restype = None
        lib.oracle_set_num_threads.argtypes = [i32]
        lib.oracle_philox_words.restype = None
        lib.oracle_philox_words.argtypes = [u64, u64, P, i64, i64, P]
        lib.oracle_philox_block.restype = None
        lib.oracle_philox_block.argtypes = [P, u32, u32, P]
        lib.oracle_noise_at.restype = None
        lib.oracle_noise_at.argtypes = [u64, u64, u32, i64, i32, P, P, P]
        lib.oracle_noise_row.restype = None
        lib.oracle_noise_row.argtypes = [u64, u64, u32, i64, i32, P]
        lib.oracle_noise_of_uniform.restype = None
        lib.oracle_noise_of_uniform.argtypes = [ctypes.c_double, P, P]
        lib.oracle_noise_grid.restype = None
        lib.oracle_noise_grid.argtypes = [i32, u64, i64, P, P]
        lib.oracle_logits.restype = None
        lib.oracle_logits.argtypes = [P, P, i64, i64, i64, P]
        lib.oracle_sample_fused.restype = None
        lib.oracle_sample_fused.argtypes = [P, P, i64, i64, i64, P, P, u64, u64, P,
                                            i32, P, P, P]
        lib.oracle_e4m3_to_double.restype = ctypes.c_double
        lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_logits_w8.restype = None
        lib.oracle_logits_w8.argtypes = [P, P, P, i64, i64, i64, P]
        lib.oracle_sample_fused_w8.restype = None
        lib.oracle_sample_fused_w8.argtypes = [P, P, P, i64, i64, i64, P, P, u64, u64, P,
                                               i32, P, P, P]
        lib.oracle_e2m1_to_double.restype = ctypes.c_double
        lib.oracle_e2m1_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_e8m0_to_double.restype = ctypes.c_double
        lib.oracle_e8m0_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_logits_w4.restype = None
        lib.oracle_logits_w4.argtypes = [P, P, P, i64, i64, i64, P]
        lib.oracle_sample_fused_w4.restype = None
        lib.oracle_sample_fused_w4.argtypes = [P, P, P, i64, i64, i64, P, P, u64, u64, P, i32, P,
                                               P, P]
        lib.oracle_sample_fused_topk.restype = None
        lib.oracle_sample_fused_topk.argtypes = [P, P, i64, i64, i64, P, P, u64, u64, P, i32,
                                                 i32, P, P]
        lib.oracle_sample_logits_topk.restype = None
        lib.oracle_sample_logits_topk.argtypes = [P, i64, i64, P, u64, u64, P, i32, i32, P, P]
        lib.oracle_topk_repeated_row.restype = None
        lib.oracle_topk_repeated_row.argtypes = [P, i64, ctypes.c_float, u64, u64, P, i64,
                                                 i32, i32, P]
        lib.oracle_sample_logits.restype = None
        lib.oracle_sample_logits.argtypes = [P, i64, i64, P, u64, u64, P, i32, P, P, P]
        lib.oracle_sample_repeated_row.restype = None
        lib.oracle_sample_repeated_row.argtypes = [P, i64, ctypes.c_float, u64, u64, P,
                                                   i64, i32, P, P]
        lib.oracle_filter_kept.restype = None
        lib.oracle_filter_kept.argtypes = [P, i64, i64, P, P, P, P, P, P]
        lib.oracle_sample_fused_filtered.restype = None
        lib.oracle_sample_fused_filtered.argtypes = [P, P, i64, i64, i64, P, P, P, P, u64, u64,
                                                     P, i32, P, P, P, P]
        lib.oracle_sample_logits_filtered.restype = None
        lib.oracle_sample_logits_filtered.argtypes = [P, i64, i64, P, P, P, P, u64, u64, P, i32,
                                                      P, P, P]
        lib.oracle_filtered_repeated_row.restype = None
        lib.oracle_filtered_repeated_row.argtypes = [P, i64, ctypes.c_float, i32, ctypes.c_float,
                                                     ctypes.c_float, u64, u64, P, i64, i32, P]
        lib.oracle_repetition_penalty.restype = None
        lib.oracle_repetition_penalty.argtypes = [P, i64, i64, P, i64, P, P]
        lib.oracle_filter_logits.restype = None
        lib.oracle_filter_logits.argtypes = [P, i64, i64, P, P, P, P, P, P]
        lib.oracle_accept_uniform.restype = ctypes.c_double
        lib.oracle_accept_uniform.argtypes = [u64, u64, u32]
        lib.oracle_verify.restype = None
        lib.oracle_verify.argtypes = [P, P, P, i64, i64, i64, P, u64, u64, P, i32, P, P, P, P]
        lib.oracle_verify_repeated.restype = None
        lib.oracle_verify_repeated.argtypes = [P, P, P, i64, i64, ctypes.c_float, u64, u64, P,
                                               i64, i32, P, P]
        _lib = lib
        return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _bf16_bits(x) -> np.ndarray:
    """Accept a numpy uint16 array of bf16 bit patterns or a torch bfloat16 tensor."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint16
        return np.ascontiguousarray(x)
    import torch  # local: only the tests pass torch tensors
    assert x.dtype == torch.bfloat16
    return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def _u32_or_none(row_ids, B):
    if row_ids is None:
        return None
    a = np.ascontiguousarray(np.asarray(row_ids, dtype=np.uint32))
    assert a.shape == (B,)
    return a


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def philox_words(seed: int, offset: int, row_ids, B: int, n_ctr: int) -> np.ndarray:
    """uint32[B, n_ctr, 4]: Philox4x32-10 words of counters (j, row, offset)."""
    out = np.zeros((B, n_ctr, 4), dtype=np.uint32)
    rid = _u32_or_none(row_ids, B)
    _load().oracle_philox_words(seed, offset, _ptr(rid), B, n_ctr, _ptr(out))
    return out


def philox_block(ctr, key) -> np.ndarray:
    """The raw Philox4x32-10 bijection of counter ctr[4] under key (k0, k1)."""
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    _load().oracle_philox_block(_ptr(c), int(key[0]), int(key[1]), _ptr(out))
    return out


def noise_at(seed: int, offset: int, row_id: int, i: int, fp64: bool):
    """(u, E, g) of vocabulary index i in logical row row_id."""
    u, E, g = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _load().oracle_noise_at(seed, offset, row_id, i, int(fp64),
                            ctypes.byref(u), ctypes.byref(E), ctypes.byref(g))
    return u.value, E.value, g.value


def noise_row(seed: int, offset: int, row_id: int, V: int, fp64: bool) -> np.ndarray:
    """float64[V]: the Gumbel noise g_i of every vocabulary index of logical row row_id."""
    g = np.zeros(V, dtype=np.float64)
    _load().oracle_noise_row(seed, offset, row_id, V, int(fp64), _ptr(g))
    return g


def noise_of_uniform(u: float):
    """(E, g) for a uniform value u."""
    E, g = ctypes.c_double(), ctypes.c_double()
    _load().oracle_noise_of_uniform(float(u), ctypes.byref(E), ctypes.byref(g))
    return E.value, g.value


def noise_grid(fp64: bool, k0: int, n: int):
    """(E, g) float64 for the midpoint-grid points k0 .. k0+n-1 (23 or 52 bits)."""
    E = np.zeros(n, dtype=np.float64)
    g = np.zeros(n, dtype=np.float64)
    _load().oracle_noise_grid(int(fp64), k0, n, _ptr(E), _ptr(g))
    return E, g


def logits(H, W) -> np.ndarray:
    """float64[B, V] = H @ W.T with H[B,D], W[V,D] given as bf16."""
    h, w = _bf16_bits(H), _bf16_bits(W)
    B, D = h.shape
    V, D2 = w.shape
    assert D == D2
    Y = np.zeros((B, V), dtype=np.float64)
    _load().oracle_logits(_ptr(h), _ptr(w), B, D, V, _ptr(Y))
    return Y


def sample_fused(H, W, temp, bias=None, *, seed: int, offset: int, row_ids=None,
                 fp64_noise: bool = False):
    """(idx int64[B], gap float64[B], best float64[B]) for the fused definition."""
    h, w = _bf16_bits(H), _bf16_bits(W)
    B, D = h.shape
    V = w.shape[0]
    t = np.ascontiguousarray(np.asarray(temp, dtype=np.float32).reshape(B))
    bb = None
    if bias is not None:
        bb = np.ascontiguousarray(np.asarray(bias, dtype=np.float32))
        assert bb.shape == (B, V)
    rid = _u32_or_none(row_ids, B)
    idx = np.zeros(B, dtype=np.int64)
    gap = np.zeros(B, dtype=np.float64)
    best = np.zeros(B, dtype=np.float64)
    _load().oracle_sample_fused(_ptr(h), _ptr(w), B, D, V, _ptr(t), _ptr(bb), seed, offset,
                                _ptr(rid), int(fp64_noise), _ptr(idx), _ptr(gap), _ptr(best))
    return idx, gap, best


def e4m3_to_double(codes) -> np.ndarray:
    """float64 values of OCP FP8 E4M3 bit patterns (uint8 array)."""
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8)).reshape(-1)
    f = _load().oracle_e4m3_to_double
    return np.array([f(int(v)) for v in c], dtype=np.float64).reshape(np.shape(codes))


def logits_w8(H, W8, scale) -> np.ndarray:
    """float64[B, V] = scale[i] * (H @ e4m3(W8).T), H bf16 [B,D], W8 uint8 [V,D]."""
    h = _bf16_bits(H)
    w = np.ascontiguousarray(np.asarray(W8, dtype=np.uint8))
    sc = np.ascontiguousarray(np.asarray(scale, dtype=np.float32).reshape(-1))
    B, D = h.shape
    V, D2 = w.shape
    assert D == D2 and sc.shape[0] == V
    Y = np.zeros((B, V), dtype=np.float64)
    _load().oracle_logits_w8(_ptr(h), _ptr(w), _ptr(sc), B, D, V, _ptr(Y))
    return Y


def sample_fused_w8(H, W8, scale, temp, bias=None, *, seed: int, offset: int, row_ids=None,
                    fp64_noise: bool = False):
    """(idx, gap, best) for the fused definition over FP8 E4M3 weights with one
    float32 scale per vocabulary row."""
    h = _bf16_bits(H)
    w = np.ascontiguousarray(np.asarray(W8, dtype=np.uint8))
    sc = np.ascontiguousarray(np.asarray(scale, dtype=np.float32).reshape(-1))
    B, D = h.shape
    V = w.shape[0]
    assert w.shape[1] == D and sc.shape[0] == V
    t = np.ascontiguousarray(np.asarray(temp, dtype=np.float32).reshape(B))
    bb = None
    if bias is not None:
        bb = np.ascontiguousarray(np.asarray(bias, dtype=np.float32))
        assert bb.shape == (B, V)
    rid = _u32_or_none(row_ids, B)
    idx = np.zeros(B, dtype=np.int64)
    gap = np.zeros(B, dtype=np.float64)
    best = np.zeros(B, dtype=np.float64)
    _load().oracle_sample_fused_w8(_ptr(h), _ptr(w), _ptr(sc), B, D, V, _ptr(t), _ptr(bb), seed,
                                   offset, _ptr(rid), int(fp64_noise), _ptr(idx), _ptr(gap),
                                   _ptr(best))
    return idx, gap, best


def sample_logits(logits_f32, temp, *, seed: int, offset: int, row_ids=None,
                  fp64_noise: bool = False):
    """(idx, gap, best) for the standalone sampler over float32 logits[B,V]."""
    x = np.ascontiguousarray(np.asarray(logits_f32, dtype=np.float32))
    B, V = x.shape
    t = np.ascontiguousarray(np.asarray(temp, dtype=np.float32).reshape(B))
    rid = _u32_or_none(row_ids, B)
    idx = np.zeros(B, dtype=np.int64)
    gap = np.zeros(B, dtype=np.float64)
    best = np.zeros(B, dtype=np.float64)
    _load().oracle_sample_logits(_ptr(x), B, V, _ptr(t), seed, offset, _ptr(rid),
                                 int(fp64_noise), _ptr(idx), _ptr(gap), _ptr(best))
    return idx, gap, best


def e2m1_to_double(codes) -> np.ndarray:
    """float64 values of FP4 E2M1 codes (low 4 bits of each uint8)."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    lib = _load()
    return np.array([lib.oracle_e2m1_to_double(int(v)) for v in c], dtype=np.float64)


def e8m0_to_double(codes) -> np.ndarray:
    """float64 values of E8M0 scale codes."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    lib = _load()
    return np.array([lib.oracle_e8m0_to_double(int(v)) for v in c], dtype=np.float64)


def logits_w4(H, W4, S) -> np.ndarray:
    """float64[B, V] over MXFP4 weights: W4 uint8 [V, D/2] (element 2j in the low
    nibble of byte j), S uint8 [V, D/32] E8M0 block scales."""
    h = _bf16_bits(H)
    w = np.ascontiguousarray(np.asarray(W4, dtype=np.uint8))
    sc = np.ascontiguousarray(np.asarray(S, dtype=np.uint8))
    B, D = h.shape
    V = w.shape[0]
    assert D % 32 == 0 and w.shape == (V, D // 2) and sc.shape == (V, D // 32)
    Y = np.zeros((B, V), dtype=np.float64)
    _load().oracle_logits_w4(_ptr(h), _ptr(w), _ptr(sc), B, D, V, _ptr(Y))
    return Y


def sample_fused_w4(H, W4, S, temp, bias=None, *, seed: int, offset: int, row_ids=None,
                    fp64_noise: bool = False):
    """(idx, gap, best) for the fused definition over MXFP4 weights."""
    h = _bf16_bits(H)
    w = np.ascontiguousarray(np.asarray(W4, dtype=np.uint8))
    sc = np.ascontiguousarray(np.asarray(S, dtype=np.uint8))
    B, D = h.shape
    V = w.shape[0]
    assert D % 32 == 0 and w.shape == (V, D // 2) and sc.shape == (V, D // 32)
    t = np.ascontiguousarray(np.asarray(temp, dtype=np.float32).reshape(B))
    bb = None
    if bias is not None:
        bb = np.ascontiguousarray(np.asarray(bias, dtype=np.float32))
        assert bb.shape == (B, V)
    rid = _u32_or_none(row_ids, B)
    idx = np.zeros(B, dtype=np.int64)
    gap = np.zeros(B, dtype=np.float64)
    best = np.zeros(B, dtype=np.float64)
    _load().oracle_sample_fused_w4(_ptr(h), _ptr(w), _ptr(sc), B, D, V, _ptr(t), _ptr(bb), seed,
                                   offset, _ptr(rid), int(fp64_noise), _ptr(idx), _ptr(gap),
                                   _ptr(best))
    return idx, gap, best


def sample_fused_topk(H, W, temp, bias=None, *, k: int, seed: int, offset: int, row_ids=None,
                      fp64_noise: bool = False):
    """(idx [B, k], top [B, k + 1]) for Gumbel-top-k over the fused definition:
    the k largest perturbed scores' indices, largest first (-1 past the valid
    ones), and the k + 1 largest scores (-inf past the valid ones)."""
    h = _bf16_bits(H)
    w = _bf16_bits(W)
    B, D = h.shape
    V = w.shape[0]
    assert w.shape[1] == D and k >= 1
    t = np.ascontiguousarray(np.asarray(temp, dtype=np.float32).reshape(B))
    bb = None
    if bias is not None:
        bb = np.ascontiguousarray(np.asarray(bias, dtype=np.float32))
        assert bb.shape == (B, V)
    rid = _u32_or_none(row_ids, B)
    idx = np.zeros((B, k), dtype=np.int64)
    top = np.zeros((B, k + 1), dtype=np.float64)
    _load().oracle_sample_fused_topk(_ptr(h), _ptr(w), B, D, V, _ptr(t), _ptr(bb), seed, offset,
                                     _ptr(rid), int(fp64_noise), k, _ptr(idx), _ptr(top))
    return idx, top


def sample_logits_topk(logits_f32, temp, *, k: int, seed: int, offset: int, row_ids=None,
                       fp64_noise: bool = False):
    """(idx [B, k], top [B, k + 1]) for Gumbel-top-k over float32 logits[B,V]."""
    x = np.ascontiguousarray(np.asarray(logits_f32, dtype=np.float32))
    B, V = x.shape
    assert k >= 1
    t = np.ascontiguousarray(np.asarray(temp, dtype=np.float32).reshape(B))
    rid = _u32_or_none(row_ids, B)
    idx = np.zeros((B, k), dtype=np.int64)
    top = np.zeros((B, k + 1), dtype=np.float64)
    _load().oracle_sample_logits_topk(_ptr(x), B, V, _ptr(t), seed, offset, _ptr(rid),
                                      int(fp64_noise), k, _ptr(idx), _ptr(top))
    return idx, top


def topk_repeated_row(row_f32, temp: float, *, k: int, seed: int, offset: int, row_ids,
                      fp64_noise: bool = False):
    """idx [n, k]: Gumbel-top-k of one logits row under n logical row ids."""
    x = np.ascontiguousarray(np.asarray(row_f32, dtype=np.float32).reshape(-1))
    rid = np.ascontiguousarray(np.asarray(row_ids, dtype=np.uint32).reshape(-1))
    idx = np.zeros((rid.shape[0], k), dtype=np.int64)
    _load().oracle_topk_repeated_row(_ptr(x), x.shape[0], float(temp), seed, offset, _ptr(rid),
                                     rid.shape[0], int(fp64_noise), k, _ptr(idx))
    return idx


def sample_repeated_row(row_f32, temp: float, *, seed: int, offset: int, row_ids,
                        fp64_noise: bool = False, with_gap: bool = False):
    """Sampled indices of many logical rows that all carry the logits row_f32[V]
    (and their top-2 gaps if with_gap)."""
    x = np.ascontiguousarray(np.asarray(row_f32, dtype=np.float32).reshape(-1))
    rid = np.ascontiguousarray(np.asarray(row_ids, dtype=np.uint32).reshape(-1))
    out = np.zeros(rid.shape[0], dtype=np.int64)
    gap = np.zeros(rid.shape[0], dtype=np.float64) if with_gap else None
    _load().oracle_sample_repeated_row(_ptr(x), x.shape[0], float(temp), seed, offset,
                                       _ptr(rid), rid.shape[0], int(fp64_noise), _ptr(out),
                                       _ptr(gap))
    return (out, gap) if with_gap else out


def _filter_args(B, top_k, top_p, min_p):
    """Per-row filter arrays (or None when a filter is off for every row)."""
    def arr(v, dt):
        if v is None:
            return None
        a = np.asarray(v, dtype=dt)
        if a.ndim == 0:
            a = np.full(B, a, dtype=dt)
        a = np.ascontiguousarray(a.reshape(B))
        return a
    return arr(top_k, np.int32), arr(top_p, np.float32), arr(min_p, np.float32)


def filter_kept(logits_f32, temp, *, top_k=None, top_p=None, min_p=None):
    """(kept bool[B, V], margin float64[B]): the kept set of the filter chain
    temperature -> top-k -> top-p -> min-p on each row, and each row's smallest
    relative distance of a top-p or min-p decision from its boundary.  top_k,
    top_p, min_p: a scalar for every row, a per-row array, or None (off)."""
    x = np.ascontiguousarray(np.asarray(logits_f32, dtype=np.float32))
    B, V = x.shape
    t = np.ascontiguousarray(np.asarray(temp, dtype=np.float32).reshape(B))
    k, p, m = _filter_args(B, top_k, top_p, min_p)
    kept = np.zeros((B, V), dtype=np.uint8)
    margin = np.zeros(B, dtype=np.float64)
    _load().oracle_filter_kept(_ptr(x), B, V, _ptr(t), _ptr(k), _ptr(p), _ptr(m), _ptr(kept),
                               _ptr(margin))
    return kept.astype(bool), margin


def repetition_penalty(logits_f32, prev_tokens, penalty) -> np.ndarray:
    """float32[B, V]: logits with the repetition penalty applied to the tokens of
    prev_tokens[B, L] (entries outside [0, V) are padding); penalty scalar or [B]."""
    x = np.ascontiguousarray(np.asarray(logits_f32, dtype=np.float32))
    B, V = x.shape
    prev = np.ascontiguousarray(np.asarray(prev_tokens, dtype=np.int64).reshape(B, -1))
    pen = np.ascontiguousarray(np.broadcast_to(np.asarray(penalty, dtype=np.float32), (B,)).copy())
    out = np.empty_like(x)
    _load().oracle_repetition_penalty(_ptr(x), B, V, _ptr(prev), prev.shape[1], _ptr(pen), _ptr(out))
    return out


def filter_logits(logits_f32, temp, *, top_k=None, top_p=None, min_p=None):
    """(out float64[B, V], margin float64[B]): the filter chain's masked,
    temperature-scaled logits (y / t on the kept tokens, -inf elsewhere)."""
    x = np.ascontiguousarray(np.asarray(logits_f32, dtype=np.float32))
    B, V = x.shape
    t = np.ascontiguousarray(np.asarray(temp, dtype=np.float32).reshape(B))
    k, p, m = _filter_args(B, top_k, top_p, min_p)
    out = np.zeros((B, V), dtype=np.float64)
    margin = np.zeros(B, dtype=np.float64)
    _load().oracle_filter_logits(_ptr(x), B, V, _ptr(t), _ptr(k), _ptr(p), _ptr(m), _ptr(out),
                                 _ptr(margin))
    return out, margin


def sample_logits_filtered(logits_f32, temp, *, top_k=None, top_p=None, min_p=None, seed: int,
                           offset: int, row_ids=None, fp64_noise: bool = False):
    """(idx, gap, margin): filtered exact sampling over float32 logits[B,V]."""
    x = np.ascontiguousarray(np.asarray(logits_f32, dtype=np.float32))
    B, V = x.shape
    t = np.ascontiguousarray(np.asarray(temp, dtype=np.float32).reshape(B))
    k, p, m = _filter_args(B, top_k, top_p, min_p)
    rid = _u32_or_none(row_ids, B)
    idx = np.zeros(B, dtype=np.int64)
    gap = np.zeros(B, dtype=np.float64)
    margin = np.zeros(B, dtype=np.float64)
    _load().oracle_sample_logits_filtered(_ptr(x), B, V, _ptr(t), _ptr(k), _ptr(p), _ptr(m),
                                          seed, offset, _ptr(rid), int(fp64_noise), _ptr(idx),
                                          _ptr(gap), _ptr(margin))
    return idx, gap, margin


def sample_fused_filtered(H, W, temp, *, top_k=None, top_p=None, min_p=None, seed: int,
                          offset: int, row_ids=None, fp64_noise: bool = False):
    """(idx, gap, margin, vmargin): filtered exact sampling of the logits H W^T
    (H[B,D], W[V,D] bf16, summed in float64): the filter chain over those
    logits, then the fused draw over the kept tokens.  margin: the smallest
    relative distance of a top-p or min-p decision from its boundary; vmargin:
    the smallest logit gap at a top-k or top-p cut."""
    h, w = _bf16_bits(H), _bf16_bits(W)
    B, D = h.shape
    V = w.shape[0]
    t = np.ascontiguousarray(np.asarray(temp, dtype=np.float32).reshape(B))
    k, p, m = _filter_args(B, top_k, top_p, min_p)
    rid = _u32_or_none(row_ids, B)
    idx = np.zeros(B, dtype=np.int64)
    gap = np.zeros(B, dtype=np.float64)
    margin = np.zeros(B, dtype=np.float64)
    vmargin = np.zeros(B, dtype=np.float64)
    _load().oracle_sample_fused_filtered(_ptr(h), _ptr(w), B, D, V, _ptr(t), _ptr(k), _ptr(p),
                                         _ptr(m), seed, offset, _ptr(rid), int(fp64_noise),
                                         _ptr(idx), _ptr(gap), _ptr(margin), _ptr(vmargin))
    return idx, gap, margin, vmargin


def filtered_repeated_row(row_f32, temp: float, *, top_k: int = 0, top_p: float = 1.0,
                          min_p: float = 0.0, seed: int, offset: int, row_ids,
                          fp64_noise: bool = False):
    """Filtered draws of many logical rows that all carry the logits row_f32[V]."""
    x = np.ascontiguousarray(np.asarray(row_f32, dtype=np.float32).reshape(-1))
    rid = np.ascontiguousarray(np.asarray(row_ids, dtype=np.uint32).reshape(-1))
    out = np.zeros(rid.shape[0], dtype=np.int64)
    _load().oracle_filtered_repeated_row(_ptr(x), x.shape[0], float(temp), int(top_k),
                                         float(top_p), float(min_p), seed, offset, _ptr(rid),
                                         rid.shape[0], int(fp64_noise), _ptr(out))
    return out


def accept_uniform(seed: int, pos: int, row_id: int) -> float:
    """The acceptance uniform of verification position `pos` (offset + i) of
    logical row `row_id`."""
    return float(_load().oracle_accept_uniform(seed, pos, row_id))


def verify(target_f32, draft_f32, tokens, temp, *, seed: int, offset: int, row_ids=None,
           fp64_noise: bool = False):
    """(accept_len int64[B], out int64[B, K+1], margin float64[B], gap float64[B]):
    speculative-decoding verification of draft tokens[B, K] against target
    logits[B, K+1, V] and draft logits[B, K, V] (float32)."""
    tg = np.ascontiguousarray(np.asarray(target_f32, dtype=np.float32))
    dr = np.ascontiguousarray(np.asarray(draft_f32, dtype=np.float32))
    B, K1, V = tg.shape
    K = K1 - 1
    assert dr.shape == (B, K, V)
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64).reshape(B, K))
    t = np.ascontiguousarray(np.broadcast_to(np.asarray(temp, dtype=np.float32), (B,)).copy())
    rid = _u32_or_none(row_ids, B)
    acc = np.zeros(B, dtype=np.int64)
    out = np.zeros((B, K + 1), dtype=np.int64)
    margin = np.zeros(B, dtype=np.float64)
    gap = np.zeros(B, dtype=np.float64)
    _load().oracle_verify(_ptr(tg), _ptr(dr), _ptr(tok), B, K, V, _ptr(t), seed, offset,
                          _ptr(rid), int(fp64_noise), _ptr(acc), _ptr(out), _ptr(margin),
                          _ptr(gap))
    return acc, out, margin, gap


def verify_repeated(target_f32, draft_f32, tokens, temp: float, *, seed: int, offset: int,
                    row_ids, fp64_noise: bool = False):
    """(accept_len, out) for many logical rows sharing one target block
    [K+1, V] and one draft block [K, V], with draft tokens[n, K] and ids
    row_ids[n]."""
    tg = np.ascontiguousarray(np.asarray(target_f32, dtype=np.float32))
    dr = np.ascontiguousarray(np.asarray(draft_f32, dtype=np.float32))
    K1, V = tg.shape
    K = K1 - 1
    assert dr.shape == (K, V)
    rid = np.ascontiguousarray(np.asarray(row_ids, dtype=np.uint32).reshape(-1))
    n = rid.shape[0]
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64).reshape(n, K))
    acc = np.zeros(n, dtype=np.int64)
    out = np.zeros((n, K + 1), dtype=np.int64)
    _load().oracle_verify_repeated(_ptr(tg), _ptr(dr), _ptr(tok), K, V, float(temp), seed,
                                   offset, _ptr(rid), n, int(fp64_noise), _ptr(acc), _ptr(out))
    return acc, out
