"""Build libfa.so in-tree with hipcc for gfx950.

    python -m exact_io_aware_46_amd.build

Objects go to exact_io_aware_46_amd/_build/, the library to exact_io_aware_46_amd/libfa.so.
The bench's matrix-core probe (csrc/mfma_peak.hip) is built beside it as libmfma_peak.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
PEAK_LIB = os.path.join(PKG, "libmfma_peak.so")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_bwd_rk.hip", "fa_bwd_rk_drop.hip",
           "fa_fwd_fp8.hip", "fa_noalloc.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
# -packed-fp32-ops: keep the device compiler from forming packed fp32 instructions.
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Options for one source only: the one-wave dK/dV kernel's instances without dropout form
# their matrix products in VGPRs (the compiler otherwise keeps S and dP in accumulation
# registers and copies each element out before the elementwise work).
SOURCE_FLAGS = {"fa_bwd_rk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *SOURCE_FLAGS.get(src, []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, out, extra=()):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, *extra]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        objs = list(ex.map(_compile, SOURCES + ["mfma_peak.hip"]))
    _link(objs[:-1], LIB, [f"-Wl,--version-script={os.path.join(CSRC, 'libfa.map')}"])
    _link(objs[-1:], PEAK_LIB)
    if verbose:
        print(f"built {LIB} and {PEAK_LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
