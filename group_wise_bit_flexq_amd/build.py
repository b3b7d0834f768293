"""Build libflexq.so (the HIP kernels and the C ABI of include/flexq.h) for gfx950.

Every csrc/*.hip file is compiled to an object with hipcc and every csrc/*.cpp file
(host-only code) with ROCm's clang++, in parallel, and the objects are linked into
group_wise_bit_flexq_amd/libflexq.so.  Objects go to _build/ at the repository root.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libflexq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = os.environ.get("FLEXQ_CXX", "/opt/rocm/llvm/bin/clang++")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
    # no packed-fp32 instructions anywhere in the library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# host-only code: x86-64-v3 (AVX2, FMA, F16C) and no floating-point contraction, so the
# quantizer's code decisions see the same fp32 operations as the GPU's
HOST_CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-march=x86-64-v3", "-ffp-contract=off",
    "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{INCLUDE}",
]


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


# per-source additions: decode attention's K pass accumulates one small MFMA chain per
# token step and reads it at once, so its accumulators belong in ordinary VGPRs
# (the default heuristic puts them in AGPRs and copies them back every step)
EXTRA_CFLAGS = {"attn_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    base, ext = os.path.splitext(os.path.basename(src))
    obj = os.path.join(BUILD, base + (".o" if ext == ".hip" else ".host.o"))
    if ext == ".hip":
        cmd = [HIPCC, *CFLAGS, *EXTRA_CFLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    else:
        cmd = [CLANGXX, *HOST_CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
