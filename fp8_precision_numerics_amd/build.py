"""Build libfp8mi.so (the HIP/CDNA4 kernels and the C ABI) in-tree for gfx950.

    python -m fp8_precision_numerics_amd.build        # or: from ... import build_library

Each HIP source is compiled to an object with hipcc (in parallel), then linked
into ``fp8_precision_numerics_amd/lib/libfp8mi.so``.  Compilation flags:
  * ``--offload-arch=gfx950``: CDNA4 only;
  * ``-O3`` without fast-math, so fp32 division stays correctly rounded (the
    scale rule needs it) and fp32 denormals are kept;
  * ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed-fp32
    instructions are generated;
  * ``-mcode-object-version=5``: loadable by every ROCm runtime that PyTorch
    may bring along (the library binds to the HIP runtime already in the
    process when torch is imported first).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIBPATH = os.path.join(LIBDIR, "libfp8mi.so")
BUILDDIR = os.path.join(ROOT, "_build")

SOURCES = ["api.hip", "quantize.hip", "amax_update.hip", "gemm.hip", "gemm_requant.hip", "grouped_gemm.hip", "allreduce.hip", "mx.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
         "-mcode-object-version=5",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libfp8mi")


# Per-source additions.  grouped_gemm.hip: matrix-core results in ordinary
# VGPRs instead of accumulation registers.  The exact grouped kernel promotes
# each 128-deep partial into a separate running sum with a VALU multiply-add;
# with the partials in accumulation registers every promotion first copies
# them out (64 extra VALU instructions per step and wave), which made that
# kernel VALU-bound (measured on MI355X: 943-949 us -> 875-910 us on the MoE
# shape, identical results).
EXTRA_FLAGS = {"grouped_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILDDIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *EXTRA_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build_library(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source and link libfp8mi.so; returns the library path."""
    os.makedirs(BUILDDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIBPATH + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIBPATH)
    return LIBPATH


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
