"""Build the W4A8 MoE HIP library (libw4a8moe.so) for gfx950, in-tree.

    python -m quantized_grouped_gemm_token_amd.build        # or build() below

Every source in csrc/ is compiled by hipcc for --offload-arch=gfx950 and
linked into one shared library next to this file.  Flags:
  * -O3, C++17, position independent;
  * packed fp32 instructions disabled (-packed-fp32-ops) for every kernel;
  * fp32 division and square root correctly rounded (the FP8 codes are
    bit-exact only with IEEE division);
  * MFMA results kept in VGPRs (the GEMMs scale every MFMA result on the
    VALU right away, which cannot read accumulation registers).
"""
from __future__ import annotations

import glob
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
LIB = os.path.join(PKG, "libw4a8moe.so")
ARCH = "gfx950"
C_CALLER_SRC = os.path.join(ROOT, "tests", "c_caller", "moe_layer.cpp")
C_CALLER = os.path.join(ROOT, "tests", "c_caller", "moe_layer")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", src, "-o", obj] + COMMON
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    if os.path.exists(C_CALLER_SRC):
        build_c_caller(verbose)
    return LIB


def build_c_caller(verbose: bool = True) -> str:
    """The native test caller (host code only, linked against the library with a relative rpath)."""
    tmp = C_CALLER + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O2", "-std=c++17", "-Wall", f"-I{INCLUDE}", C_CALLER_SRC,
           "-o", tmp, f"-L{PKG}", "-lw4a8moe", "-Wl,-rpath,$ORIGIN/../../quantized_grouped_gemm_token_amd"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build of the native caller failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, C_CALLER)
    if verbose:
        print(f"built {C_CALLER}", file=sys.stderr)
    return C_CALLER


if __name__ == "__main__":
    build()
