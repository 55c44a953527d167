"""Build libfa.so (the HIP kernels and their C ABI) in-tree for gfx950.

    python -m exact_io_aware_52_amd.build_lib

Objects go to ``_build/`` at the repository root; the shared library is
written next to this file.  Every call recompiles.
"""

import hashlib
import json
import os
import re
import shutil
import struct
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
# Race-check build: the same sources with every LDS ring stage fenced
# (FA_SERIALIZE_STAGES); its results must equal libfa.so's bit for bit.
SERIAL_LIB = os.path.join(PKG, "libfa_serial.so")
# Step timeline build: the forward with FA_STEP_STAMPS (per-step clock stamps
# of chosen work-groups, read by bench.py --step-stamps), the rest as libfa.so.
STAMPS_LIB = os.path.join(PKG, "libfa_stamps.so")
# Unit-rate build: instruction-rate kernels (matrix products, exponentials,
# fp32 fma/add, bf16 packing, and their overlap) for the step cost model,
# read by bench.py --unit-rates; no attention code.
RATES_LIB = os.path.join(PKG, "libfa_rates.so")
# Hash of each kernel's gfx950 machine code (all instances of one kernel
# template together), written at every build.  Counter summaries under
# profiles/ carry the hash of the code they were taken on, and the bench
# reports their traffic only while it matches.
CODE_MANIFEST = os.path.join(PKG, "kernel_code.json")
KERNELS = ("fa_fwd_kernel", "fa_fwd_keys_kernel", "fa_fwd_kgroups_kernel", "fa_fwd_combine_kernel",
           "fa_bwd_dq_kernel", "fa_bwd_dkdv_kernel")

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


def _compile(src, variant=""):
    out_dir = os.path.join(BUILD, variant) if variant else BUILD
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    flags = list(COMMON)
    if src in NO_VGPR_FORM:
        i = flags.index("-amdgpu-mfma-vgpr-form=1")
        del flags[i - 1:i + 1]
    if variant == "serial":
        flags.append("-DFA_SERIALIZE_STAGES")
    if variant == "stamps":
        flags.append("-DFA_STEP_STAMPS")
    cmd = [hipcc()] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    return obj, err


def _link(objects, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + list(objects)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, lib)


def _llvm(tool):
    exe = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", tool)
    if not os.path.exists(exe):
        raise RuntimeError(f"{exe} not found")
    return exe


def _elf_functions(path):
    """{symbol: machine-code bytes} of the FUNC symbols of an ELF64 file."""
    data = open(path, "rb").read()
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    secs = [struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize) for i in range(shnum)]
    # (name, type, flags, addr, offset, size, link, info, align, entsize)
    out = {}
    for sec in secs:
        if sec[1] != 2:          # SHT_SYMTAB
            continue
        strtab = secs[sec[6]]
        for off in range(sec[4], sec[4] + sec[5], 24):
            name_off, info, _, shndx, value, size = struct.unpack_from("<IBBHQQ", data, off)
            if info & 0xF != 2 or size == 0 or shndx >= shnum:   # STT_FUNC with code
                continue
            end = data.index(b"\0", strtab[4] + name_off)
            name = data[strtab[4] + name_off:end].decode()
            text = secs[shndx]
            start = text[4] + (value - text[3])
            out[name] = data[start:start + size]
    return out


def kernel_code_hashes(objects):
    """sha256 (16 hex digits) of each kernel template's gfx950 code, over all
    its instances (key: the kernel name), and of each instance alone (key:
    "instance:" + its mangled name), from the device code objects bundled in
    the objects."""
    funcs = {}
    tmp = os.path.join(BUILD, "code")
    os.makedirs(tmp, exist_ok=True)
    for obj in objects:
        base = os.path.join(tmp, os.path.splitext(os.path.basename(obj))[0])
        r = subprocess.run([_llvm("llvm-objcopy"), f"--dump-section=.hip_fatbin={base}.fatbin",
                            obj], capture_output=True, text=True)
        if r.returncode != 0:
            continue             # host-only object (the C ABI layer)
        subprocess.run([_llvm("clang-offload-bundler"), "--unbundle", "--type=o",
                        f"--input={base}.fatbin", f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}",
                        f"--output={base}.co"], check=True, capture_output=True)
        funcs.update(_elf_functions(base + ".co"))
    hashes = {}
    for kern in KERNELS:
        h = hashlib.sha256()
        names = sorted(n for n in funcs if re.search(rf"\d{kern}I", n))
        for n in names:
            h.update(n.encode())
            h.update(funcs[n])
            # each instance on its own as well: a counter summary names the
            # instance it was taken on, which other instances do not change
            hashes["instance:" + n] = hashlib.sha256(n.encode() + funcs[n]).hexdigest()[:16]
        hashes[kern] = h.hexdigest()[:16] if names else None
    return hashes


def build(verbose=False):
    """Compile libfa.so, the race-check build libfa_serial.so, the step
    timeline build libfa_stamps.so and the unit-rate library libfa_rates.so."""
    for var in ("serial", "stamps", "rates"):
        os.makedirs(os.path.join(BUILD, var), exist_ok=True)
    jobs = ([(src, "") for src in SOURCES] + [(src, "serial") for src in SOURCES] +
            [("fa_fwd.hip", "stamps"), ("fa_rates.hip", "rates")])
    with ThreadPoolExecutor(max_workers=min(9, len(jobs))) as ex:
        results = list(ex.map(lambda j: _compile(*j), jobs))
    for obj, err in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
    main = [o for (o, _), (_, var) in zip(results, jobs) if not var]
    serial = [o for (o, _), (_, var) in zip(results, jobs) if var == "serial"]
    stamps_fwd = [o for (o, _), (_, var) in zip(results, jobs) if var == "stamps"]
    rates = [o for (o, _), (_, var) in zip(results, jobs) if var == "rates"]
    _link(main, LIB)
    _link(serial, SERIAL_LIB)
    _link([o for o in main if not o.endswith("fa_fwd.o")] + stamps_fwd, STAMPS_LIB)
    _link(rates, RATES_LIB)
    hashes = kernel_code_hashes(main)
    with open(CODE_MANIFEST, "w") as fh:
        json.dump(hashes, fh, indent=1, sort_keys=True)
    if verbose:
        print(f"built {LIB}, {SERIAL_LIB}, {STAMPS_LIB} and {RATES_LIB}")
        print(f"kernel code hashes: { {k: v for k, v in hashes.items() if ':' not in k} }")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
