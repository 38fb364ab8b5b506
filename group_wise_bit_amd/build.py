"""Build libqlin.so in-tree with hipcc for gfx950.

    python -m group_wise_bit_amd.build          # or: import and call build()

The library is plain HIP C++ behind a C ABI (include/qlin.h); no PyTorch
extension machinery is involved.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libqlin.so")
SOURCES = [os.path.join(CSRC, "qlin_api.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("device_common.h", "codes.h", "kernels.h")] + [
    os.path.join(ROOT, "include", "qlin.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU ops stay off (compiler-generated v_pk_*_f32 excluded)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqlin)")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile libqlin.so (always recompiles).  Returns the library path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
