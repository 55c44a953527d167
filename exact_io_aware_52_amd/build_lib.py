"""Build libfa.so (the HIP kernels and their C ABI) in-tree for gfx950.

    python -m exact_io_aware_52_amd.build_lib

Objects go to ``_build/`` at the repository root; the shared library is
written next to this file.  Every call recompiles.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_bwd_f32.hip"]
# Sources compiled without the VGPR-form matrix-core option.  fp32 backward:
# with it, LLVM's "Rewrite AGPR-Copy-MFMA" pass crashes.  16-bit backward: the
# d = 128 dK/dV pass (one wave per SIMD, 474 registers) keeps its dK and dV
# accumulators in AGPRs; in VGPR form the compiler copies them between the
# two register files around every product (~150 copies per step against 64
# AGPR reads of the softmax without it; 7% faster without).  The other
# backward kernels measure the same either way.
NO_VGPR_FORM = {"fa_bwd_f32.hip", "fa_bwd.hip"}
ARCH = "gfx950"

# Packed fp32 VALU instructions are switched off for all device code.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # Matrix-core accumulators in ordinary VGPRs (the softmax reads them
          # directly; no copies between accumulation and vector registers).
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          # fp32 instances cannot meet the two-waves-per-SIMD request; that is
          # expected (they exist for accuracy, not speed).
          "-Wall", "-Wno-unused-function", "-Wno-pass-failed", "-I", INCLUDE, "-I", CSRC]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")
    return exe


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    flags = list(COMMON)
    if src in NO_VGPR_FORM:
        i = flags.index("-amdgpu-mfma-vgpr-form=1")
        del flags[i - 1:i + 1]
    cmd = [hipcc()] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    return obj, err


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for obj, err in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
