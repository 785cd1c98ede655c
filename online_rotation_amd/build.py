"""Build librq.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

Usage: python -m online_rotation_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librq.so")
SOURCES = ["rq_api.cpp", "rotate_quant.hip", "kron.hip", "gemm_w4a4.hip", "gemm_ra.hip",
           "gemm_decode.hip", "gemm_decode8.hip", "kv_quant.hip", "quant8.hip",
           "clip_search.hip"]
ARCH = "gfx950"

# Packed-fp32 instructions are disabled for all device code.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# MFMA accumulators in VGPRs (no AGPR copies) for the kernels listed here.
# gemm_ra.hip and kron.hip are built without the flag; held to 256 registers
# by their two-wavefronts-per-SIMD bound, they get VGPR accumulators from the
# compiler as well (their code uses no AGPRs).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA_FLAGS = {"rotate_quant.hip": VGPR_FORM, "gemm_w4a4.hip": VGPR_FORM, "gemm_decode.hip": VGPR_FORM,
               "gemm_decode8.hip": VGPR_FORM}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def _compile(hipcc: str, src: str, objdir: str, verbose: bool) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-x", "hip", "-I", os.path.join(ROOT, "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source (in parallel) and link librq.so; returns the library path."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    hipcc = _hipcc()
    jobs = jobs or max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(hipcc, src, objdir, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
