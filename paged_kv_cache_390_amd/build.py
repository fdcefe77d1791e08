"""Build libpa.so in-tree: HIP kernels for gfx950 with hipcc, host C++ with
g++, linked by hipcc.  Run directly (``python -m paged_kv_cache_390_amd.build``)
or through ``__graft_entry__.build()``."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpa.so")

ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")
HIP_SOURCES = ["decode.hip", "decode_gqa.hip", "prefill.hip", "cache_ops.hip", "bench_read.hip", "validate.hip"]
CXX_SOURCES = ["block_manager.cpp", "status.cpp"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler away from packed fp32 ALU forms on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
# per-source extra hipcc flags: the matrix-core attention kernels keep their
# accumulators in VGPRs (the online softmax reads and rescales them every tile;
# in AGPRs each access would add a copy)
HIP_EXTRA = {"decode_gqa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
             "prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; ROCm is required to build libpa.so")
    return p


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    if verbose and r.stdout.strip():
        print(r.stdout, flush=True)


def build(verbose: bool = False, extra_hip_flags=()) -> str:
    os.makedirs(OBJ, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        o = os.path.join(OBJ, src + ".o")
        objs.append(o)
        jobs.append([hipcc, *HIPCC_FLAGS, *HIP_EXTRA.get(src, []), *extra_hip_flags, "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", o])
    for src in CXX_SOURCES:
        o = os.path.join(OBJ, src + ".o")
        objs.append(o)
        jobs.append(["g++", *CXX_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", o])
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    tmp = LIB + f".tmp{os.getpid()}"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp, "-lpthread"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
