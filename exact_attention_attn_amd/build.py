"""Build libattn.so (the HIP kernels and the C ABI of include/attn.h) for gfx950.

Usage: ``python -m exact_attention_attn_amd.build`` or ``build()`` from Python.  The
library is written next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_decode.hip", "attn_kvcache.hip", "attn_bwd.hip"]
ARCH = "gfx950"

# Per-source extra flags.  The backward keeps its dK / dV accumulators in AGPRs through
# inline asm and the other MFMA results in VGPRs (-amdgpu-mfma-vgpr-form), where VALU
# reads them.
EXTRA_FLAGS = {"attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

# Packed fp32 VALU ops are kept out of the generated code (-packed-fp32-ops).  The
# direct-to-LDS loads are inline asm that writes M0 and so lists it as clobbered; clang
# flags every such statement (-Winline-asm: M0 is reserved to the compiler, which sets it
# right before each use of its own), hence -Wno-inline-asm.
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-inline-asm",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: cannot build libattn.so")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPFLAGS, *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise and verbose:
        print("\n".join(noise), file=sys.stderr)
    return obj


# The hardware-rate measurement (MFMA / VALU / LDS issue rates on one SIMD) behind the
# forward kernel's roofline discussion: a separate executable, not part of the library.
HW_RATES_SRC = "hw_rates.hip"
HW_RATES = os.path.join(HERE, "hw_rates")


def build_hw_rates(verbose: bool = False) -> str:
    cmd = [hipcc(), *HIPFLAGS, os.path.join(CSRC, HW_RATES_SRC), "-o", HW_RATES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {HW_RATES_SRC} failed:\n{r.stdout}\n{r.stderr}")
    return HW_RATES


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES) + 1) as ex:
        hw = ex.submit(build_hw_rates, verbose)
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
        hw.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libattn.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
