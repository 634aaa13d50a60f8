"""Builds libpbq.so in-tree: HIP kernels with hipcc for gfx950, the host C++
with g++, linked by hipcc.  Run as ``python -m paged_block_quantized_amd.build``
or call ``build()``."""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libpbq.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_SOURCES = ["quantize_store.hip", "paged_attn.hip", "copy_blocks.hip", "swap_blocks.hip", "stream_read.hip", "scratch.hip"]
CPP_SOURCES = ["capi.cpp", "pool.cpp"]

# -packed-fp32-ops: no packed fp32 VALU instructions are generated.
# -ffp-contract=off: every fused multiply-add in the kernels is written out.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
             "-ffp-contract=off", "-fno-fast-math", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]
CPP_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__",
             "-I", os.path.join(ROCM, "include"), "-I", INCLUDE, "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, extra_hip_flags=(), out=LIB, build_dir=BUILD):
    """Compile every source and link libpbq.so (always rebuilds).  ``out`` and
    ``build_dir`` let variants with other compile-time settings be built
    beside the default library."""
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    cxx = shutil.which("g++") or "g++"
    os.makedirs(build_dir, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        jobs.append([hipcc, *HIP_FLAGS, *extra_hip_flags, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CPP_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        jobs.append([cxx, *CPP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [j[-1] for j in jobs]
    tmp = out + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
