"""Exact categorical sampling fused into the LM head, for AMD MI355X (gfx950).

Thin Python binding over ``libfsample.so`` (C ABI in ``include/fsample.h``).
Every step of the sampling path runs in the library's HIP kernels; this module
only checks tensor arguments, finds the current HIP stream, keeps a workspace
per (device, stream), and passes raw pointers.  PyTorch provides device memory
and streams.  If the library has not been built, every call raises.

    tok = sample_fused(H, W, temp, bias=None, seed=1234, offset=step)   # [B] int64
    tok = sample_fused_w8(H, W8, w_scale, temp, seed=1234, offset=step)  # FP8 E4M3 W
    tok = sample_logits(logits, temp, seed=1234, offset=step, fp64_noise=True)
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "FS_FP64_NOISE", "FS_TOPK_MAX", "FSampleError", "sample_fused", "sample_fused_noalloc",
    "sample_fused_w8",
    "sample_fused_topk", "sample_fused_mxfp4", "sample_logits", "sample_logits_topk",
    "sample_logits_filtered", "sample_fused_filtered", "workspace_bytes", "debug_logits_mxfp4",
    "debug_philox_words",
    "debug_logits", "debug_logits_w8", "debug_noise", "library_path", "load_library",
    "KernelTimer",
    "fused_tiles",
    "debug_stream_read",
]

FS_FP64_NOISE = 0x1
FS_TOPK_MAX = 8
_STATUS = {0: "FS_OK", 1: "FS_ERR_INVALID_ARG", 2: "FS_ERR_UNSUPPORTED", 3: "FS_ERR_WORKSPACE",
           4: "FS_ERR_HIP"}

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libfsample.so")
_lib = None
_lock = threading.Lock()
_workspaces: dict = {}


class FSampleError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {detail}")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libfsample.so (after torch, so both share one HIP runtime)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built: run `python __graft_entry__.py` "
                               "or decode_exact_categorical_amd.build.build()")
        lib = ctypes.CDLL(_LIB_PATH)
        P, i64, u64, u32, sz, i32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                     ctypes.c_uint32, ctypes.c_size_t, ctypes.c_int)
        lib.fs_workspace_bytes.restype = sz
        lib.fs_workspace_bytes.argtypes = [i64, i64, u32]
        lib.fs_sample_fused.restype = i32
        lib.fs_sample_fused.argtypes = [P, P, i64, i64, i64, P, P, u64, u64, P, P, u32, P, sz, P]
        lib.fs_sample_logits.restype = i32
        lib.fs_sample_logits.argtypes = [P, i64, i64, P, u64, u64, i32, P, P, P, sz, P]
        lib.fs_status_string.restype = ctypes.c_char_p
        lib.fs_status_string.argtypes = [i32]
        lib.fs_last_error.restype = ctypes.c_char_p
        lib.fs_last_error.argtypes = []
        lib.fs_debug_philox_words.restype = i32
        lib.fs_debug_philox_words.argtypes = [u64, u64, P, i64, i64, P, P]
        lib.fs_profile_begin.restype = i32
        lib.fs_profile_begin.argtypes = []
        lib.fs_profile_end.restype = i32
        lib.fs_profile_end.argtypes = [P, P]
        lib.fs_profile_end_detail.restype = i32
        lib.fs_profile_end_detail.argtypes = [P, P, P, P, i64]
        lib.fs_workspace_bytes_fused_filtered.restype = sz
        lib.fs_workspace_bytes_fused_filtered.argtypes = [i64, i64]
        lib.fs_sample_fused_filtered.restype = i32
        lib.fs_sample_fused_filtered.argtypes = [P, P, i64, i64, i64, P, P, P, P, u64, u64, P, P,
                                                 u32, P, sz, P]
        lib.fs_sample_fused_noalloc.restype = i32
        lib.fs_sample_fused_noalloc.argtypes = [P, P, i64, i64, i64, P, P, u64, u64, P, P, u32, P]
        lib.fs_fused_tiles.restype = i32
        lib.fs_fused_tiles.argtypes = [i64, i64, i64, i32]
        lib.fs_debug_stream_read.restype = i32
        lib.fs_debug_stream_read.argtypes = [P, sz, P, P]
        lib.fs_debug_noise.restype = i32
        lib.fs_debug_noise.argtypes = [P, i64, i32, P, P, P]
        lib.fs_debug_logits.restype = i32
        lib.fs_debug_logits.argtypes = [P, P, i64, i64, i64, P, P]
        lib.fs_workspace_bytes_topk.restype = sz
        lib.fs_workspace_bytes_topk.argtypes = [i64, i64, u32]
        lib.fs_sample_fused_topk.restype = i32
        lib.fs_sample_fused_topk.argtypes = [P, P, i64, i64, i64, P, P, u64, u64, i32, P, P, u32,
                                             P, sz, P]
        lib.fs_sample_logits_topk.restype = i32
        lib.fs_sample_logits_topk.argtypes = [P, i64, i64, P, u64, u64, i32, i32, P, P, P, sz, P]
        lib.fs_sample_fused_mxfp4.restype = i32
        lib.fs_sample_fused_mxfp4.argtypes = [P, P, P, i64, i64, i64, P, P, u64, u64, P, P, u32, P,
                                              sz, P]
        lib.fs_debug_logits_mxfp4.restype = i32
        lib.fs_debug_logits_mxfp4.argtypes = [P, P, P, i64, i64, i64, P, P]
        lib.fs_sample_fused_w8.restype = i32
        lib.fs_sample_fused_w8.argtypes = [P, P, P, i64, i64, i64, P, P, u64, u64, P, P, u32, P,
                                           sz, P]
        lib.fs_debug_logits_w8.restype = i32
        lib.fs_sample_logits_filtered.restype = i32
        lib.fs_sample_logits_filtered.argtypes = [P, i64, i64, P, P, P, P, u64, u64, i32, P, P, P,
                                                  sz, P]
        lib.fs_workspace_bytes_filtered.restype = sz
        lib.fs_workspace_bytes_filtered.argtypes = [i64, i64]
        lib.fs_repetition_penalty.restype = i32
        lib.fs_repetition_penalty.argtypes = [P, i64, i64, P, i64, P, P, P]
        lib.fs_filter_logits.restype = i32
        lib.fs_filter_logits.argtypes = [P, i64, i64, P, P, P, P, P, P]
        lib.fs_verify.restype = i32
        lib.fs_verify.argtypes = [P, P, P, i64, i64, i64, P, u64, u64, i32, P, P, P, P, sz, P]
        lib.fs_workspace_bytes_verify.restype = sz
        lib.fs_workspace_bytes_verify.argtypes = [i64, i64, i64]
        lib.fs_debug_logits_w8.argtypes = [P, P, P, i64, i64, i64, P, P]
        _lib = lib
        return lib


def _check(status: int, fn: str):
    if status != 0:
        detail = load_library().fs_last_error().decode(errors="replace")
        raise FSampleError(status, fn, detail)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, device, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _temp_tensor(temp, B: int, device) -> torch.Tensor:
    if isinstance(temp, (int, float)):
        return _constant(float(temp), torch.float32, B, device)
    _need(temp, "temp", torch.float32, device, (B,))
    return temp


def _row_ids(row_ids, B: int, device):
    if row_ids is None:
        return None
    if row_ids.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
        raise TypeError("row_ids must be int32 (read as uint32)")
    _need(row_ids, "row_ids", row_ids.dtype, device, (B,))
    return row_ids


def workspace_bytes(B: int, V: int, fp64_noise: bool = False) -> int:
    return int(load_library().fs_workspace_bytes(B, V, FS_FP64_NOISE if fp64_noise else 0))


def _workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """A cached uint8 workspace for the current stream of `device` (stream-ordered reuse).
    Zero-filled when allocated, as the library requires; each call leaves it zeroed."""
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def sample_fused(H: torch.Tensor, W: torch.Tensor, temp, bias: torch.Tensor | None = None, *,
                 seed: int, offset: int, row_ids: torch.Tensor | None = None,
                 fp64_noise: bool = False, out: torch.Tensor | None = None) -> torch.Tensor:
    """One exact draw per row from softmax((H W^T + bias) / temp); [B] int64 (-1: no token)."""
    lib = load_library()
    dev = H.device
    if dev.type != "cuda":
        raise ValueError("H must be a GPU tensor")
    if H.dim() != 2 or W.dim() != 2:
        raise ValueError("H must be [B, D] and W [V, D]")
    B, D = H.shape
    V = W.shape[0]
    _need(H, "H", torch.bfloat16, dev, (B, D))
    _need(W, "W", torch.bfloat16, dev, (V, D))
    t = _temp_tensor(temp, B, dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, dev, (B, V))
    rid = _row_ids(row_ids, B, dev)
    if out is None:
        out = torch.empty((B,), dtype=torch.int64, device=dev)
    _need(out, "out", torch.int64, dev, (B,))
    flags = FS_FP64_NOISE if fp64_noise else 0
    need = int(lib.fs_workspace_bytes(B, V, flags)) if V > 0 else 0
    ws = _workspace(dev, need)
    st = lib.fs_sample_fused(_ptr(H), _ptr(W), B, D, V, _ptr(t), _ptr(bias), seed, offset,
                             _ptr(out), _ptr(rid), flags, _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "fs_sample_fused")
    return out


def sample_fused_noalloc(H: torch.Tensor, W: torch.Tensor, temp, bias: torch.Tensor | None = None,
                         *, seed: int, offset: int, row_ids: torch.Tensor | None = None,
                         fp64_noise: bool = False, out: torch.Tensor | None = None) -> torch.Tensor:
    """sample_fused without a workspace: the library's built-in per-GPU scratch
    (B <= 1024; calls that overlap on one GPU race on it).  `out` given, the
    call allocates nothing."""
    lib = load_library()
    dev = H.device
    if dev.type != "cuda":
        raise ValueError("H must be a GPU tensor")
    if H.dim() != 2 or W.dim() != 2:
        raise ValueError("H must be [B, D] and W [V, D]")
    B, D = H.shape
    V = W.shape[0]
    _need(H, "H", torch.bfloat16, dev, (B, D))
    _need(W, "W", torch.bfloat16, dev, (V, D))
    _need(temp, "temp", torch.float32, dev, (B,))
    if bias is not None:
        _need(bias, "bias", torch.float32, dev, (B, V))
    rid = _row_ids(row_ids, B, dev)
    if out is None:
        out = torch.empty((B,), dtype=torch.int64, device=dev)
    _need(out, "out", torch.int64, dev, (B,))
    flags = FS_FP64_NOISE if fp64_noise else 0
    st = lib.fs_sample_fused_noalloc(_ptr(H), _ptr(W), B, D, V, _ptr(temp), _ptr(bias), seed,
                                     offset, _ptr(out), _ptr(rid), flags, _stream(dev))
    _check(st, "fs_sample_fused_noalloc")
    return out


def _w8_bytes(W8: torch.Tensor, dev, V: int, D: int) -> torch.Tensor:
    """FP8 E4M3 weights as their uint8 codes (a float8_e4m3fn tensor is viewed)."""
    if W8.dtype == torch.float8_e4m3fn:
        W8 = W8.view(torch.uint8)
    _need(W8, "W8", torch.uint8, dev, (V, D))
    return W8


def sample_fused_w8(H: torch.Tensor, W8: torch.Tensor, w_scale: torch.Tensor, temp,
                    bias: torch.Tensor | None = None, *, seed: int, offset: int,
                    row_ids: torch.Tensor | None = None, fp64_noise: bool = False,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """sample_fused with FP8 E4M3 weights: row i of W is w_scale[i] * e4m3(W8[i]).
    W8 is [V, D] uint8 codes or float8_e4m3fn; w_scale [V] float32."""
    lib = load_library()
    dev = H.device
    if dev.type != "cuda":
        raise ValueError("H must be a GPU tensor")
    if H.dim() != 2 or W8.dim() != 2:
        raise ValueError("H must be [B, D] and W8 [V, D]")
    B, D = H.shape
    V = W8.shape[0]
    _need(H, "H", torch.bfloat16, dev, (B, D))
    W8 = _w8_bytes(W8, dev, V, D)
    _need(w_scale, "w_scale", torch.float32, dev, (V,))
    t = _temp_tensor(temp, B, dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, dev, (B, V))
    rid = _row_ids(row_ids, B, dev)
    if out is None:
        out = torch.empty((B,), dtype=torch.int64, device=dev)
    _need(out, "out", torch.int64, dev, (B,))
    flags = FS_FP64_NOISE if fp64_noise else 0
    need = int(lib.fs_workspace_bytes(B, V, flags)) if V > 0 else 0
    ws = _workspace(dev, need)
    st = lib.fs_sample_fused_w8(_ptr(H), _ptr(W8), _ptr(w_scale), B, D, V, _ptr(t), _ptr(bias),
                                seed, offset, _ptr(out), _ptr(rid), flags, _ptr(ws), ws.numel(),
                                _stream(dev))
    _check(st, "fs_sample_fused_w8")
    return out


def _mxfp4_args(H, W4, w4_scale, dev):
    B, D = H.shape
    V = W4.shape[0]
    _need(H, "H", torch.bfloat16, dev, (B, D))
    _need(W4, "W4", torch.uint8, dev, (V, D // 2))
    _need(w4_scale, "w4_scale", torch.uint8, dev, (V, D // 32))
    return B, D, V


def sample_fused_mxfp4(H: torch.Tensor, W4: torch.Tensor, w4_scale: torch.Tensor, temp,
                       bias: torch.Tensor | None = None, *, seed: int, offset: int,
                       row_ids: torch.Tensor | None = None, fp64_noise: bool = False,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """sample_fused with MXFP4 weights: W4 uint8 [V, D/2] E2M1 codes (element 2j in
    the low nibble of byte j), w4_scale uint8 [V, D/32] E8M0 block scales."""
    lib = load_library()
    dev = H.device
    if dev.type != "cuda":
        raise ValueError("H must be a GPU tensor")
    B, D, V = _mxfp4_args(H, W4, w4_scale, dev)
    t = _temp_tensor(temp, B, dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, dev, (B, V))
    rid = _row_ids(row_ids, B, dev)
    if out is None:
        out = torch.empty((B,), dtype=torch.int64, device=dev)
    _need(out, "out", torch.int64, dev, (B,))
    flags = FS_FP64_NOISE if fp64_noise else 0
    need = int(lib.fs_workspace_bytes(B, V, flags)) if V > 0 else 0
    ws = _workspace(dev, need)
    st = lib.fs_sample_fused_mxfp4(_ptr(H), _ptr(W4), _ptr(w4_scale), B, D, V, _ptr(t), _ptr(bias),
                                   seed, offset, _ptr(out), _ptr(rid), flags, _ptr(ws), ws.numel(),
                                   _stream(dev))
    _check(st, "fs_sample_fused_mxfp4")
    return out


def sample_logits(logits: torch.Tensor, temp, *, seed: int, offset: int,
                  row_ids: torch.Tensor | None = None, fp64_noise: bool = False,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """One exact draw per row from softmax(logits / temp) over float32 logits [B, V]."""
    lib = load_library()
    dev = logits.device
    if dev.type != "cuda":
        raise ValueError("logits must be a GPU tensor")
    if logits.dim() != 2:
        raise ValueError("logits must be [B, V]")
    B, V = logits.shape
    _need(logits, "logits", torch.float32, dev, (B, V))
    t = _temp_tensor(temp, B, dev)
    rid = _row_ids(row_ids, B, dev)
    if out is None:
        out = torch.empty((B,), dtype=torch.int64, device=dev)
    _need(out, "out", torch.int64, dev, (B,))
    need = int(lib.fs_workspace_bytes(B, V, FS_FP64_NOISE if fp64_noise else 0)) if V > 0 else 0
    ws = _workspace(dev, need)
    st = lib.fs_sample_logits(_ptr(logits), B, V, _ptr(t), seed, offset, int(bool(fp64_noise)),
                              _ptr(out), _ptr(rid), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "fs_sample_logits")
    return out


_constants: dict = {}


def _constant(v, dtype, B: int, device) -> torch.Tensor:
    """A [B] tensor holding the scalar v on `device`, made once per (value,
    dtype, B, device) and reused (the library only reads it), so a scalar
    parameter costs no fill kernel per call."""
    key = (float(v), dtype, B, device.index)
    t = _constants.get(key)
    if t is None:
        if len(_constants) > 256:
            _constants.clear()
        t = torch.full((B,), v, dtype=dtype, device=device)
        _constants[key] = t
    return t


def _filter_param(v, name: str, dtype, B: int, device):
    """A per-row filter parameter: None (off), a Python scalar for every row, or
    a [B] tensor of `dtype` on the device."""
    if v is None:
        return None
    if isinstance(v, (int, float)):
        return _constant(v, dtype, B, device)
    _need(v, name, dtype, device, (B,))
    return v


def sample_logits_filtered(logits: torch.Tensor, temp, *, top_k=None, top_p=None, min_p=None,
                           seed: int, offset: int, row_ids: torch.Tensor | None = None,
                           fp64_noise: bool = False,
                           out: torch.Tensor | None = None) -> torch.Tensor:
    """One exact draw per row from softmax(logits / temp) restricted to the kept set of
    the filters top-k, top-p, min-p (applied in that order) over float32 logits [B, V].
    top_k (int32), top_p, min_p (float32): None, a scalar, or a [B] tensor."""
    lib = load_library()
    dev = logits.device
    if dev.type != "cuda":
        raise ValueError("logits must be a GPU tensor")
    if logits.dim() != 2:
        raise ValueError("logits must be [B, V]")
    B, V = logits.shape
    _need(logits, "logits", torch.float32, dev, (B, V))
    t = _temp_tensor(temp, B, dev)
    k = _filter_param(top_k, "top_k", torch.int32, B, dev)
    p = _filter_param(top_p, "top_p", torch.float32, B, dev)
    m = _filter_param(min_p, "min_p", torch.float32, B, dev)
    rid = _row_ids(row_ids, B, dev)
    if out is None:
        out = torch.empty((B,), dtype=torch.int64, device=dev)
    _need(out, "out", torch.int64, dev, (B,))
    need = int(lib.fs_workspace_bytes_filtered(B, V)) if V > 0 else 0
    ws = _workspace(dev, need) if need > 0 else None
    st = lib.fs_sample_logits_filtered(_ptr(logits), B, V, _ptr(t), _ptr(k), _ptr(p), _ptr(m),
                                       seed, offset, int(bool(fp64_noise)), _ptr(out), _ptr(rid),
                                       _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev))
    _check(st, "fs_sample_logits_filtered")
    return out


def sample_fused_filtered(H: torch.Tensor, W: torch.Tensor, temp, *, top_k=None, top_p=None,
                          min_p=None, seed: int, offset: int, row_ids: torch.Tensor | None = None,
                          fp64_noise: bool = False,
                          out: torch.Tensor | None = None) -> torch.Tensor:
    """Filtered exact sampling fused into the LM head: per row, the draw
    sample_logits_filtered makes over the float32 logits H W^T, without writing
    them (a row the tiles' lists cannot resolve is computed again and drawn
    exactly inside the same call).  top_k (int32), top_p, min_p (float32):
    None, a scalar, or a [B] tensor."""
    lib = load_library()
    dev = H.device
    if dev.type != "cuda":
        raise ValueError("H must be a GPU tensor")
    if H.dim() != 2 or W.dim() != 2:
        raise ValueError("H must be [B, D] and W [V, D]")
    B, D = H.shape
    V = W.shape[0]
    _need(H, "H", torch.bfloat16, dev, (B, D))
    _need(W, "W", torch.bfloat16, dev, (V, D))
    t = _temp_tensor(temp, B, dev)
    k = _filter_param(top_k, "top_k", torch.int32, B, dev)
    p = _filter_param(top_p, "top_p", torch.float32, B, dev)
    m = _filter_param(min_p, "min_p", torch.float32, B, dev)
    rid = _row_ids(row_ids, B, dev)
    if out is None:
        out = torch.empty((B,), dtype=torch.int64, device=dev)
    _need(out, "out", torch.int64, dev, (B,))
    need = int(lib.fs_workspace_bytes_fused_filtered(B, V)) if V > 0 else 0
    ws = _workspace(dev, need)
    st = lib.fs_sample_fused_filtered(_ptr(H), _ptr(W), B, D, V, _ptr(t), _ptr(k), _ptr(p),
                                      _ptr(m), seed, offset, _ptr(out), _ptr(rid),
                                      FS_FP64_NOISE if fp64_noise else 0, _ptr(ws), ws.numel(),
                                      _stream(dev))
    _check(st, "fs_sample_fused_filtered")
    return out


def repetition_penalty(logits: torch.Tensor, prev_tokens: torch.Tensor, penalty, *,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """Logits [B, V] float32 with the repetition penalty applied to the tokens of
    prev_tokens [B, L] int64 (entries outside [0, V) are padding): y * penalty where
    y < 0, y / penalty elsewhere.  penalty: a float or a [B] tensor; out may be logits."""
    lib = load_library()
    dev = logits.device
    if dev.type != "cuda":
        raise ValueError("logits must be a GPU tensor")
    if logits.dim() != 2 or prev_tokens.dim() != 2:
        raise ValueError("logits must be [B, V] and prev_tokens [B, L]")
    B, V = logits.shape
    L = prev_tokens.shape[1]
    _need(logits, "logits", torch.float32, dev, (B, V))
    _need(prev_tokens, "prev_tokens", torch.int64, dev, (B, L))
    pen = _temp_tensor(penalty, B, dev)
    if out is None:
        out = torch.empty_like(logits)
    _need(out, "out", torch.float32, dev, (B, V))
    st = lib.fs_repetition_penalty(_ptr(logits), B, V, _ptr(prev_tokens) if L > 0 else None, L,
                                   _ptr(pen), _ptr(out), _stream(dev))
    _check(st, "fs_repetition_penalty")
    return out


_penalise = repetition_penalty  # `sample` takes an argument of that name


def sample(logits: torch.Tensor, temperature, *, top_k=None, top_p=None, min_p=None,
           repetition_penalty=None, prev_tokens: torch.Tensor | None = None, seed: int,
           offset: int, row_ids: torch.Tensor | None = None, fp64_noise: bool = False):
    """The spec-decode-ops sample pipeline: repetition penalty (when repetition_penalty
    and prev_tokens are given), temperature, top-k, top-p, min-p, then the exact draw.
    One int64 token per row."""
    x = logits
    if repetition_penalty is not None and prev_tokens is not None:
        x = _penalise(logits, prev_tokens, repetition_penalty)
    return sample_logits_filtered(x, temperature, top_k=top_k, top_p=top_p, min_p=min_p,
                                  seed=seed, offset=offset, row_ids=row_ids,
                                  fp64_noise=fp64_noise)


def filter_logits(logits: torch.Tensor, temp, *, top_k=None, top_p=None, min_p=None,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """The filter chain's output over float32 logits [B, V] (top-k, top-p, min-p after
    temperature): y / temp where the chain keeps a token, -inf where it drops one."""
    lib = load_library()
    dev = logits.device
    if dev.type != "cuda":
        raise ValueError("logits must be a GPU tensor")
    if logits.dim() != 2:
        raise ValueError("logits must be [B, V]")
    B, V = logits.shape
    _need(logits, "logits", torch.float32, dev, (B, V))
    t = _temp_tensor(temp, B, dev)
    k = _filter_param(top_k, "top_k", torch.int32, B, dev)
    p = _filter_param(top_p, "top_p", torch.float32, B, dev)
    m = _filter_param(min_p, "min_p", torch.float32, B, dev)
    if out is None:
        out = torch.empty((B, V), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, (B, V))
    if out.data_ptr() == logits.data_ptr() and B * V > 0:
        raise ValueError("out may not alias logits")
    st = lib.fs_filter_logits(_ptr(logits), B, V, _ptr(t), _ptr(k), _ptr(p), _ptr(m), _ptr(out),
                              _stream(dev))
    _check(st, "fs_filter_logits")
    return out


def verify(target_logits: torch.Tensor, draft_logits: torch.Tensor, draft_tokens: torch.Tensor,
           temp, *, seed: int, offset: int, row_ids: torch.Tensor | None = None,
           fp64_noise: bool = False, accept_len: torch.Tensor | None = None,
           out: torch.Tensor | None = None):
    """Speculative-decoding verification: (accept_len int64 [B], out int64 [B, K+1]).
    target_logits float32 [B, K+1, V], draft_logits float32 [B, K, V], draft_tokens int64
    [B, K]; out[b, :accept_len[b] + 1] are the emitted tokens, distributed as the target's
    own draws; offset is the absolute position of the first draft token."""
    lib = load_library()
    dev = target_logits.device
    if dev.type != "cuda":
        raise ValueError("target_logits must be a GPU tensor")
    if target_logits.dim() != 3 or target_logits.shape[1] < 1:
        raise ValueError("target_logits must be [B, K+1, V]")
    B, K1, V = target_logits.shape
    K = K1 - 1
    _need(target_logits, "target_logits", torch.float32, dev, (B, K + 1, V))
    _need(draft_logits, "draft_logits", torch.float32, dev, (B, K, V))
    _need(draft_tokens, "draft_tokens", torch.int64, dev, (B, K))
    t = _temp_tensor(temp, B, dev)
    rid = _row_ids(row_ids, B, dev)
    if accept_len is None:
        accept_len = torch.empty((B,), dtype=torch.int64, device=dev)
    if out is None:
        out = torch.empty((B, K + 1), dtype=torch.int64, device=dev)
    _need(accept_len, "accept_len", torch.int64, dev, (B,))
    _need(out, "out", torch.int64, dev, (B, K + 1))
    need = int(lib.fs_workspace_bytes_verify(B, K, V))
    ws = _workspace(dev, need)
    st = lib.fs_verify(_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), B, K, V,
                       _ptr(t), seed, offset, int(bool(fp64_noise)), _ptr(accept_len), _ptr(out),
                       _ptr(rid), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "fs_verify")
    return accept_len, out


def sample_fused_topk(H: torch.Tensor, W: torch.Tensor, temp, bias: torch.Tensor | None = None, *,
                      k: int, seed: int, offset: int, row_ids: torch.Tensor | None = None,
                      fp64_noise: bool = False, out: torch.Tensor | None = None) -> torch.Tensor:
    """Gumbel-top-k fused into the LM head: k draws without replacement per row from
    softmax((H W^T + bias) / temp); [B, k] int64, largest perturbed score first."""
    lib = load_library()
    dev = H.device
    if dev.type != "cuda":
        raise ValueError("H must be a GPU tensor")
    if H.dim() != 2 or W.dim() != 2:
        raise ValueError("H must be [B, D] and W [V, D]")
    B, D = H.shape
    V = W.shape[0]
    _need(H, "H", torch.bfloat16, dev, (B, D))
    _need(W, "W", torch.bfloat16, dev, (V, D))
    t = _temp_tensor(temp, B, dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, dev, (B, V))
    rid = _row_ids(row_ids, B, dev)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int64, device=dev)
    _need(out, "out", torch.int64, dev, (B, k))
    flags = FS_FP64_NOISE if fp64_noise else 0
    need = int(lib.fs_workspace_bytes_topk(B, V, flags)) if V > 0 else 0
    ws = _workspace(dev, need)
    st = lib.fs_sample_fused_topk(_ptr(H), _ptr(W), B, D, V, _ptr(t), _ptr(bias), seed, offset, k,
                                  _ptr(out), _ptr(rid), flags, _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "fs_sample_fused_topk")
    return out


def sample_logits_topk(logits: torch.Tensor, temp, *, k: int, seed: int, offset: int,
                       row_ids: torch.Tensor | None = None, fp64_noise: bool = False,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """Gumbel-top-k: k draws without replacement per row from softmax(logits / temp),
    the indices of the k largest perturbed scores, largest first; [B, k] int64
    (-1 past a row's valid scores)."""
    lib = load_library()
    dev = logits.device
    if dev.type != "cuda":
        raise ValueError("logits must be a GPU tensor")
    if logits.dim() != 2:
        raise ValueError("logits must be [B, V]")
    B, V = logits.shape
    _need(logits, "logits", torch.float32, dev, (B, V))
    t = _temp_tensor(temp, B, dev)
    rid = _row_ids(row_ids, B, dev)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int64, device=dev)
    _need(out, "out", torch.int64, dev, (B, k))
    flags = FS_FP64_NOISE if fp64_noise else 0
    need = int(lib.fs_workspace_bytes_topk(B, V, flags)) if V > 0 else 0
    ws = _workspace(dev, need)
    st = lib.fs_sample_logits_topk(_ptr(logits), B, V, _ptr(t), seed, offset, int(bool(fp64_noise)),
                                   k, _ptr(out), _ptr(rid), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "fs_sample_logits_topk")
    return out


class KernelTimer:
    """Context manager: summed kernel milliseconds of the sampling calls made inside
    it (one launch per call), from HIP events the library records on each call's
    stream.  With per_call=True it also keeps each call's kernel milliseconds
    (`launch_ms`) and the milliseconds from each call's start to the next one's
    (`start_to_start_ms`, one fewer)."""

    _CAP = 4096

    def __init__(self, per_call: bool = False):
        self.per_call = per_call

    def __enter__(self):
        _check(load_library().fs_profile_begin(), "fs_profile_begin")
        self.kernel_ms = 0.0
        self.calls = 0
        self.launch_ms = []
        self.start_to_start_ms = []
        return self

    def __exit__(self, *exc):
        a, n = ctypes.c_double(), ctypes.c_int64()
        if not self.per_call:
            _check(load_library().fs_profile_end(ctypes.byref(a), ctypes.byref(n)),
                   "fs_profile_end")
            self.kernel_ms, self.calls = a.value, n.value
            return False
        lm = (ctypes.c_float * self._CAP)()
        ss = (ctypes.c_float * self._CAP)()
        _check(load_library().fs_profile_end_detail(ctypes.byref(a), ctypes.byref(n), lm, ss,
                                                    self._CAP), "fs_profile_end_detail")
        self.kernel_ms, self.calls = a.value, n.value
        k = min(self.calls, self._CAP)
        self.launch_ms = list(lm[:k])
        self.start_to_start_ms = list(ss[:max(0, k - 1)])
        return False


def fused_tiles(B: int, D: int, V: int, weight_format: str = "bf16") -> int:
    """Vocabulary tiles the fused calls use for (B, D, V) on the current device."""
    fmt = {"bf16": 0, "fp8": 1, "mxfp4": 2}[weight_format]
    n = int(load_library().fs_fused_tiles(B, D, V, fmt))
    if n < 0:
        raise ValueError(f"fs_fused_tiles: {load_library().fs_last_error().decode()}")
    return n


def debug_stream_read(buf: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """One plain streaming read of a contiguous device tensor (a multiple of 16
    bytes), xor-folded into out (int64 [1] on the same device)."""
    lib = load_library()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.zeros((1,), dtype=torch.int64, device=buf.device)
    _need(out, "out", torch.int64, buf.device, (1,))
    _check(lib.fs_debug_stream_read(_ptr(buf), nbytes, _ptr(out), _stream(buf.device)),
           "fs_debug_stream_read")
    return out


def debug_philox_words(seed: int, offset: int, B: int, n_ctr: int, *,
                       row_ids: torch.Tensor | None = None, device="cuda") -> torch.Tensor:
    """int32 view of the uint32 words [B, n_ctr, 4] the samplers draw from (test hook)."""
    lib = load_library()
    dev = torch.device(device)
    rid = _row_ids(row_ids, B, dev)
    out = torch.empty((B, n_ctr, 4), dtype=torch.int32, device=dev)
    _check(lib.fs_debug_philox_words(seed, offset, _ptr(rid), B, n_ctr, _ptr(out), _stream(dev)),
           "fs_debug_philox_words")
    return out


def debug_noise(words: torch.Tensor, fp64_noise: bool = False):
    """(E, g) float64 tensors the kernels derive from int32 `words` (uint32 bits):
    one word per variate, or two consecutive words with float64 noise (test hook)."""
    lib = load_library()
    dev = words.device
    _need(words, "words", torch.int32, dev)
    n = words.numel() // 2 if fp64_noise else words.numel()
    E = torch.empty(n, dtype=torch.float64, device=dev)
    g = torch.empty(n, dtype=torch.float64, device=dev)
    _check(lib.fs_debug_noise(_ptr(words), n, int(bool(fp64_noise)), _ptr(E), _ptr(g), _stream(dev)),
           "fs_debug_noise")
    return E, g


def debug_logits(H: torch.Tensor, W: torch.Tensor) -> torch.Tensor:
    """float32 [B, V] logits from the fused path's matmul code (test hook)."""
    lib = load_library()
    dev = H.device
    B, D = H.shape
    V = W.shape[0]
    _need(H, "H", torch.bfloat16, dev, (B, D))
    _need(W, "W", torch.bfloat16, dev, (V, D))
    Y = torch.empty((B, V), dtype=torch.float32, device=dev)
    _check(lib.fs_debug_logits(_ptr(H), _ptr(W), B, D, V, _ptr(Y), _stream(dev)),
           "fs_debug_logits")
    return Y


def debug_logits_w8(H: torch.Tensor, W8: torch.Tensor, w_scale: torch.Tensor) -> torch.Tensor:
    """float32 [B, V] logits from the FP8 path's matmul code and row scales (test hook)."""
    lib = load_library()
    dev = H.device
    B, D = H.shape
    V = W8.shape[0]
    _need(H, "H", torch.bfloat16, dev, (B, D))
    W8 = _w8_bytes(W8, dev, V, D)
    _need(w_scale, "w_scale", torch.float32, dev, (V,))
    Y = torch.empty((B, V), dtype=torch.float32, device=dev)
    _check(lib.fs_debug_logits_w8(_ptr(H), _ptr(W8), _ptr(w_scale), B, D, V, _ptr(Y),
                                  _stream(dev)), "fs_debug_logits_w8")
    return Y


def debug_logits_mxfp4(H: torch.Tensor, W4: torch.Tensor, w4_scale: torch.Tensor) -> torch.Tensor:
    """float32 [B, V] logits from the MXFP4 path's matmul code (test hook)."""
    lib = load_library()
    dev = H.device
    B, D, V = _mxfp4_args(H, W4, w4_scale, dev)
    Y = torch.empty((B, V), dtype=torch.float32, device=dev)
    _check(lib.fs_debug_logits_mxfp4(_ptr(H), _ptr(W4), _ptr(w4_scale), B, D, V, _ptr(Y),
                                     _stream(dev)), "fs_debug_logits_mxfp4")
    return Y
