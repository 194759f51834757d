"""Build libsa.so (HIP, gfx950) in-tree with hipcc.

Run as a script (``python structured_sparse_attention_amd/build.py``) or load this
file by path: importing it through the package would first load the library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsa.so")
SOURCES = ["sa_api.cpp", "sa_index.hip", "sa_attn.hip", "sa_decode.hip", "sa_capture.hip", "sa_sample.hip", "sa_calib.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libsa.so")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libsa.so next to this file."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed fp32 instructions are kept out of every kernel
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function",
           "-I", INCLUDE, "-I", CSRC, "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + errs)
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    # every symbol must resolve (a kernel whose host stub was not emitted shows up here, not at run time)
    import ctypes
    try:
        ctypes.CDLL(tmp, mode=os.RTLD_NOW)
    except OSError as e:
        os.unlink(tmp)
        raise RuntimeError("libsa.so does not load: %s" % e)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
