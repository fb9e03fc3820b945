"""Build libfsample.so (the gfx950 HIP kernels and the C ABI of include/fsample.h)."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfsample.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: the compiler must not emit packed fp32 VALU instructions.
FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libfsample.so (always recompiles): one hipcc
    process per source, run side by side, then one link."""
    # the host pass does not know the fp32 feature name and says so; that is harmless
    noise = "packed-fp32-ops' is not a recognized feature"
    tag = "%d" % os.getpid()
    objs, procs = [], []
    for src in sources():
        obj = os.path.join(CSRC, os.path.basename(src) + ".o" + tag)
        cmd = [HIPCC] + [f for f in FLAGS if f != "-shared"] + ["-I", INCLUDE, "-I", CSRC, "-c",
                                                                 src, "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
        objs.append(obj)
    msgs, failed = [], []
    for src, p in procs:
        out, _ = p.communicate()
        msgs += [ln for ln in out.splitlines() if noise not in ln]
        if p.returncode != 0:
            failed.append(os.path.basename(src))
    try:
        if failed:
            raise RuntimeError("hipcc failed on " + ", ".join(failed) + ":\n" + "\n".join(msgs))
        tmp = LIB + ".tmp" + tag
        res = subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs,
                             capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + res.stdout + res.stderr)
        if verbose and msgs:
            print("\n".join(msgs))
        os.replace(tmp, LIB)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
