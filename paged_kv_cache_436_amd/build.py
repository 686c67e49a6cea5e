"""Build libpkv.so in-tree for gfx950.

    python paged_kv_cache_436_amd/build.py          # build (always recompiles)

HIP sources are compiled by hipcc for --offload-arch=gfx950 with packed-fp32
instruction selection disabled; host-only C++ (pool description, block
manager, validators) by g++.  Objects go to paged_kv_cache_436_amd/_build/,
the library to paged_kv_cache_436_amd/libpkv.so, and the compute-only timing
probe to paged_kv_cache_436_amd/libpkv_probe.so.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpkv.so")
# the compute-only timing probe (include/pkv_probe.h), a library of its own
PROBE_LIB = os.path.join(HERE, "libpkv_probe.so")
PROBE_SOURCE = "compute_probe.hip"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_SOURCES = ["cache_kernels.hip", "decode_kernels.hip", "prefill_kernels.hip"]
CXX_SOURCES = ["pool.cpp", "block_manager.cpp"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core operands and results in ordinary VGPRs: without it the
    # register allocator parks accumulators and K/V buffers in AGPRs and
    # copies them back for every vector instruction that touches them
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # no combining of a wave's atomics on one address into one: the counter
    # updates are made by a single lane, and the combined form waits for the
    # atomic's result right after issuing it, which would stall the K/V
    # pipeline the decode kernel keeps in flight
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function",
]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    cxx = shutil.which("g++") or "c++"
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", os.path.join(ROCM, "include")]
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([hipcc, *HIPCC_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
    probe_obj = os.path.join(BUILD, PROBE_SOURCE + ".o")
    jobs.append([hipcc, *HIPCC_FLAGS, *inc, "-c", os.path.join(CSRC, PROBE_SOURCE), "-o", probe_obj])
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([cxx, *CXX_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", probe_obj, "-o", tmp])
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
