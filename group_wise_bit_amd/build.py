"""Build libqlin.so in-tree with hipcc for gfx950.

    python -m group_wise_bit_amd.build          # or: import and call build()

The library is plain HIP C++ behind a C ABI (include/qlin.h); no PyTorch
extension machinery is involved.  The host entry points (qlin_api.hip) and
one object per bit width and kernel family (inst.hip compiled with
-DQLIN_INST_BITS / -DQLIN_INST_PART) are compiled in parallel into _build/,
then linked into group_wise_bit_amd/libqlin.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libqlin.so")
# measurement utilities (include/qlin_peaks.h): the achieved-peak reference kernels
PEAKS_PATH = os.path.join(PKG_DIR, "libqlin_peaks.so")
PEAKS_SOURCE = os.path.join(CSRC, "peaks.hip")
API_SOURCE = os.path.join(CSRC, "qlin_api.hip")
INST_SOURCE = os.path.join(CSRC, "inst.hip")
HEADERS = [os.path.join(CSRC, f) for f in ("device_common.h", "codes.h", "kernels.h", "plan.h",
                                           "launch_impl.h")] + [
    os.path.join(ROOT, "include", "qlin.h")]

GEMV_BITS = (2, 3, 4, 5, 6, 7, 8, 16)   # part 0: GEMV and row gather (16: fp16 control)
GEMM_BITS = (2, 3, 4, 5, 6, 7, 8)       # part 1: GEMM
QUANT_BITS = (2, 3, 4, 5, 6, 7, 8)      # part 2: quantizer

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU ops stay off (compiler-generated v_pk_*_f32 excluded)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# The quantizer's arithmetic must round every operation on its own (bit-exact
# codes, scales and zero points): no a*b+c contracted into one fma.
QUANT_FLAGS = ["-ffp-contract=off"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqlin)")


def _units():
    units = [("api", API_SOURCE, [])]
    for b in GEMV_BITS:
        units.append((f"gemv_b{b}", INST_SOURCE, [f"-DQLIN_INST_BITS={b}", "-DQLIN_INST_PART=0"]))
    for b in GEMM_BITS:
        units.append((f"gemm_b{b}", INST_SOURCE, [f"-DQLIN_INST_BITS={b}", "-DQLIN_INST_PART=1"]))
    for b in QUANT_BITS:
        units.append((f"quant_b{b}", INST_SOURCE,
                      [f"-DQLIN_INST_BITS={b}", "-DQLIN_INST_PART=2", *QUANT_FLAGS]))
    return units


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n"
                           f"{res.stdout}\n{res.stderr}")
    return res.stderr


def build(verbose: bool = False, extra_flags=None, jobs: int | None = None,
          out_path: str | None = None) -> str:
    """Compile libqlin.so (always recompiles).  Returns the library path.

    extra_flags are added to every compile (host sanitizers go through
    -Xarch_host); out_path writes the library elsewhere (default in-tree)."""
    cc = hipcc()
    out_path = out_path or LIB_PATH
    obj_dir = os.path.join(BUILD_DIR, os.path.splitext(os.path.basename(out_path))[0])
    os.makedirs(obj_dir, exist_ok=True)
    flags = [*HIPCC_FLAGS, *(extra_flags or [])]
    cmds = []
    for name, src, defs in _units():
        obj = os.path.join(obj_dir, name + ".o")
        cmds.append((obj, [cc, *flags, *defs, "-c", src, "-o", obj]))
    jobs = jobs or min(16, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, cmd) for _, cmd in cmds]
        for (obj, cmd), f in zip(cmds, futs):
            err = f.result()
            if verbose:
                print(" ".join(cmd), flush=True)
                if err.strip() and "packed-fp32-ops" not in err:
                    print(err, file=sys.stderr)
    tmp = out_path + ".tmp"
    link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *(extra_flags or []),
            *[obj for obj, _ in cmds], "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    _run(link)
    os.replace(tmp, out_path)
    return out_path


def build_peaks(verbose: bool = False) -> str:
    """Compile libqlin_peaks.so (the achieved-peak reference kernels)."""
    tmp = PEAKS_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-shared", PEAKS_SOURCE, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, PEAKS_PATH)
    return PEAKS_PATH


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_peaks(verbose=True))
