"""The C ABI on the CPU: the library loads, exports every symbol include/fsample.h
declares, and rejects invalid arguments before any HIP call (so these checks
run without a GPU and launch nothing)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch  # noqa: F401  (loads the HIP runtime the library binds to)

import decode_exact_categorical_amd as fs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fsample.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fs.library_path()),
                                reason="libfsample.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fs_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = _declared()
    assert {"fs_sample_fused", "fs_sample_logits", "fs_workspace_bytes", "fs_status_string",
            "fs_last_error", "fs_debug_philox_words", "fs_debug_logits"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", fs.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\S+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = fs.load_library()
    for n in names:
        assert hasattr(lib, n)


def test_status_strings():
    lib = fs.load_library()
    for code, name in [(0, b"FS_OK"), (1, b"FS_ERR_INVALID_ARG"), (2, b"FS_ERR_UNSUPPORTED"),
                       (3, b"FS_ERR_WORKSPACE"), (4, b"FS_ERR_HIP")]:
        assert lib.fs_status_string(code).startswith(name)
    assert b"unknown" in lib.fs_status_string(99)


def test_workspace_bytes():
    lib = fs.load_library()
    assert lib.fs_workspace_bytes(0, 100, 0) > 0
    assert lib.fs_workspace_bytes(-1, 100, 0) == 0
    assert lib.fs_workspace_bytes(4, 0, 0) == 0
    assert lib.fs_workspace_bytes(4, 2**31, 0) == 0
    a = lib.fs_workspace_bytes(64, 151936, 0)
    b = lib.fs_workspace_bytes(64, 151936, fs.FS_FP64_NOISE)
    assert 64 * 256 * 8 <= a < b
    assert lib.fs_workspace_bytes(4096, 131072, 1) >= 4096 * 64 * 16


P = ctypes.c_void_p
FAKE = 0x10000  # a 16-byte-aligned non-null address; never dereferenced on these paths


def _fused(B=4, D=512, V=1000, H=FAKE, W=FAKE, temp=FAKE, out=FAKE, flags=0, ws=FAKE,
           wsb=1 << 30):
    lib = fs.load_library()
    return lib.fs_sample_fused(P(H), P(W), B, D, V, P(temp), None, 1, 0, P(out), None, flags,
                               P(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), 1), (dict(V=0), 1), (dict(V=2**31), 1), (dict(D=0), 1), (dict(D=-8), 1),
    (dict(H=0), 1), (dict(W=0), 1), (dict(temp=0), 1), (dict(out=0), 1), (dict(flags=2), 1),
    (dict(D=12), 2), (dict(H=FAKE + 4), 2), (dict(W=FAKE + 8), 2),
    (dict(ws=0), 3), (dict(wsb=16), 3), (dict(ws=FAKE + 4), 3),
])
def test_fused_rejects_before_launch(kw, code):
    assert _fused(**kw) == code
    assert fs.load_library().fs_last_error() != b""


def test_empty_batch_is_a_noop():
    lib = fs.load_library()
    assert _fused(B=0, H=0, W=0, temp=0, out=0, ws=0, wsb=0) == 0
    assert _fused(B=0) == 0
    assert lib.fs_sample_logits(None, 0, 10, None, 0, 0, 0, None, None, None, 0, None) == 0
    assert lib.fs_debug_philox_words(0, 0, None, 0, 5, None, None) == 0


def _logits(B=4, V=1000, X=FAKE, temp=FAKE, out=FAKE, fp64=0, ws=FAKE, wsb=1 << 30):
    lib = fs.load_library()
    return lib.fs_sample_logits(P(X), B, V, P(temp), 1, 0, fp64, P(out), None, P(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-2), 1), (dict(V=0), 1), (dict(V=2**31), 1), (dict(X=0), 1), (dict(temp=0), 1),
    (dict(out=0), 1), (dict(X=FAKE + 2), 2), (dict(ws=0), 3), (dict(wsb=8), 3),
    (dict(B=2**30, V=2**20), 1),
])
def test_logits_rejects_before_launch(kw, code):
    assert _logits(**kw) == code


def _filtered(B=4, V=100000, X=FAKE, temp=FAKE, out=FAKE, ws=FAKE, wsb=1 << 30):
    lib = fs.load_library()
    return lib.fs_sample_logits_filtered(P(X), B, V, P(temp), None, None, None, 1, 0, 0, P(out),
                                         None, P(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-2), 1), (dict(V=0), 1), (dict(V=2**31), 1), (dict(X=0), 1), (dict(temp=0), 1),
    (dict(out=0), 1), (dict(X=FAKE + 2), 2), (dict(B=2**31), 1),
    (dict(ws=0), 3), (dict(wsb=64), 3), (dict(ws=FAKE + 8), 3),
])
def test_filtered_rejects_before_launch(kw, code):
    assert _filtered(**kw) == code
    assert fs.load_library().fs_last_error() != b""


def test_filtered_empty_batch_is_a_noop():
    assert _filtered(B=0, X=0, temp=0, out=0, ws=0, wsb=0) == 0


def test_filtered_workspace_bytes():
    lib = fs.load_library()
    # split rows for small batches of long rows: counters, chunk headers and lists
    assert lib.fs_workspace_bytes_filtered(16, 151936) >= 16 * 19 * (8 + 512) * 8
    assert lib.fs_workspace_bytes_filtered(1, 128256) > 0
    # batches of 9 to 96 rows run the chunks and the merges as two launches
    assert lib.fs_workspace_bytes_filtered(64, 151936) >= 256 * 1024 + 64 * 19 * (8 + 512) * 8
    # one workgroup per row (large batches, short or very long rows): none
    for B, V in ((4096, 131072), (97, 151936), (16, 8192), (8, 300000), (0, 151936)):
        assert lib.fs_workspace_bytes_filtered(B, V) == 0, (B, V)
    assert lib.fs_workspace_bytes_filtered(-1, 1000) == 0
    assert lib.fs_workspace_bytes_filtered(4, 0) == 0


def test_repetition_penalty_rejects_before_launch():
    lib = fs.load_library()
    call = lambda B=4, V=100, prev=FAKE, L=3, pen=FAKE, X=FAKE, Y=FAKE: lib.fs_repetition_penalty(
        P(X), B, V, P(prev), L, P(pen), P(Y), None)
    assert call(B=-1) == 1 and call(V=0) == 1 and call(L=-1) == 1 and call(B=65536) == 1
    assert call(X=0) == 1 and call(Y=0) == 1 and call(pen=0) == 1 and call(prev=0) == 1
    assert call(X=FAKE + 2) == 2 and call(Y=FAKE + 6) == 2
    assert call(B=0, X=0, Y=0, pen=0, prev=0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), 1), (dict(V=0), 1), (dict(X=0), 1), (dict(temp=0), 1), (dict(Y=0), 1),
    (dict(X=FAKE + 2), 2), (dict(Y=FAKE + 6), 2),
])
def test_filter_logits_rejects_before_launch(kw, code):
    args = dict(B=4, V=1000, X=FAKE, temp=FAKE, Y=FAKE)
    args.update(kw)
    lib = fs.load_library()
    assert lib.fs_filter_logits(P(args["X"]), args["B"], args["V"], P(args["temp"]), None, None,
                                None, P(args["Y"]), None) == code
    assert lib.fs_filter_logits(None, 0, 10, None, None, None, None, None, None) == 0


def _verify(B=4, K=4, V=100000, T=FAKE, D=FAKE, tok=FAKE, temp=FAKE, acc=FAKE, out=FAKE,
            ws=FAKE, wsb=1 << 30):
    lib = fs.load_library()
    return lib.fs_verify(P(T), P(D), P(tok), B, K, V, P(temp), 1, 0, 0, P(acc), P(out), None,
                         P(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), 1), (dict(V=0), 1), (dict(V=2**31), 1), (dict(K=-1), 1), (dict(K=33), 1),
    (dict(B=65537), 1), (dict(T=0), 1), (dict(D=0), 1), (dict(tok=0), 1), (dict(temp=0), 1),
    (dict(acc=0), 1), (dict(out=0), 1), (dict(T=FAKE + 2), 2), (dict(D=FAKE + 6), 2),
    (dict(ws=0), 3), (dict(wsb=1024), 3), (dict(ws=FAKE + 16), 3),
])
def test_verify_rejects_before_launch(kw, code):
    assert _verify(**kw) == code
    assert fs.load_library().fs_last_error() != b""


def test_verify_sizes_and_workspace():
    lib = fs.load_library()
    assert _verify(B=0, T=0, D=0, tok=0, temp=0, acc=0, out=0, ws=0, wsb=0) == 0
    # K = 0 needs no draft rows or tokens (a plain draw from target row 0): only
    # the workspace is missing here
    assert _verify(K=0, D=0, tok=0, ws=0, wsb=0) == 3
    # the leading counter region, then the per-chunk softmax partials of 2K rows,
    # the bonus row's candidates and the residual candidates
    nC = (151936 + 2047) // 2048
    assert lib.fs_workspace_bytes_verify(64, 4, 151936) >= 256 * 1024 + 64 * nC * (8 * 16 + 16 + 16)
    assert lib.fs_workspace_bytes_verify(1, 0, 10) > 0
    for B, K, V in ((-1, 4, 100), (4, 33, 100), (4, -1, 100), (4, 4, 0), (65537, 1, 100)):
        assert lib.fs_workspace_bytes_verify(B, K, V) == 0, (B, K, V)


def test_every_workspace_keeps_its_counters_in_the_leading_region():
    """One workspace may serve every entry point in turn (the Python binding
    caches one per stream): each keeps its completion counters in the first
    256 KiB and its other data after them, so no call's data lands on another's
    counters.  The filtered sampler's split rows and verification reserve the
    whole region."""
    lib = fs.load_library()
    assert lib.fs_workspace_bytes_filtered(1, 151936) >= 256 * 1024 + 8 * 8
    assert lib.fs_workspace_bytes_verify(1, 1, 8) >= 256 * 1024
    assert lib.fs_workspace_bytes(1, 8, 0) >= 256 * 1024


def test_debug_hooks_reject_before_launch():
    lib = fs.load_library()
    assert lib.fs_debug_philox_words(0, 0, None, -1, 4, P(FAKE), None) == 1
    assert lib.fs_debug_philox_words(0, 0, None, 4, 4, None, None) == 1
    assert lib.fs_debug_philox_words(0, 0, None, 4, 4, P(FAKE + 4), None) == 2
    assert lib.fs_debug_philox_words(0, 0, None, 2**20, 2**12, P(FAKE), None) == 1
    assert lib.fs_debug_logits(P(FAKE), P(FAKE), 4, 12, 100, P(FAKE), None) == 2
    assert lib.fs_debug_logits(P(FAKE), P(FAKE), 4, 16, 100, None, None) == 1


def test_python_binding_checks_without_gpu():
    with pytest.raises(ValueError):
        fs.sample_fused(torch.zeros(2, 8, dtype=torch.bfloat16),
                        torch.zeros(3, 8, dtype=torch.bfloat16), 1.0, seed=0, offset=0)


def _noalloc(B=4, D=512, V=1000, H=FAKE, W=FAKE, temp=FAKE, out=FAKE, flags=0):
    lib = fs.load_library()
    return lib.fs_sample_fused_noalloc(P(H), P(W), B, D, V, P(temp), None, 1, 0, P(out), None,
                                       flags, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), 1), (dict(V=0), 1), (dict(D=0), 1), (dict(H=0), 1), (dict(temp=0), 1),
    (dict(out=0), 1), (dict(flags=2), 1), (dict(D=12), 2), (dict(W=FAKE + 8), 2),
    (dict(B=1025), 2),
])
def test_noalloc_rejects_before_launch(kw, code):
    # sizes past the built-in scratch (B > 1024) are refused like any other
    # argument error: on the host, before any HIP call
    assert _noalloc(**kw) == code
    assert fs.load_library().fs_last_error() != b""
