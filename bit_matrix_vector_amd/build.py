"""Builds the HIP library libqmv.so in-tree for gfx950.

    python -m bit_matrix_vector_amd.build

Compiles the kernel instantiation slices in parallel (one hipcc process per
(dtype, format family) slice), the dispatch unit, and the host API with g++,
then links them into bit_matrix_vector_amd/libqmv.so.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqmv.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    # fp32 division and square root correctly rounded (the quantizers rely on it)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep hipcc from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}",
]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
# the host API is plain C++ (g++); the public header names hipStream_t, so it
# sees the HIP runtime API header of the AMD platform
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
             f"-I{os.path.join(ROCM, 'include')}", f"-I{INCLUDE}", f"-I{CSRC}"]


def _jobs() -> list[tuple[list[str], str]]:
    jobs = []
    # the heaviest slices (affine codes) first, so the pool's tail is short
    for fam in (0, 5, 1, 2, 3, 4):
        for dt in (0, 1, 2):
            obj = os.path.join(BUILD, f"qmv_inst_{dt}_{fam}.o")
            jobs.append(([HIPCC, *HIP_FLAGS, f"-DQMV_DT={dt}", f"-DQMV_FAM={fam}", "-c",
                          os.path.join(CSRC, "qmv_inst.hip"), "-o", obj], obj))
    obj = os.path.join(BUILD, "qmv_dispatch.o")
    jobs.append(([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "qmv_dispatch.hip"), "-o", obj],
                 obj))
    for dt in (0, 1, 2):
        obj = os.path.join(BUILD, f"qmv_qvm_{dt}.o")
        jobs.append(([HIPCC, *HIP_FLAGS, f"-DQVM_DT={dt}", "-c",
                      os.path.join(CSRC, "qmv_qvm.hip"), "-o", obj], obj))
    for dt in (1, 2):
        obj = os.path.join(BUILD, f"qmv_qmm_{dt}.o")
        jobs.append(([HIPCC, *HIP_FLAGS, f"-DQMM_DT={dt}", "-c",
                      os.path.join(CSRC, "qmv_qmm.hip"), "-o", obj], obj))
    obj = os.path.join(BUILD, "qmv_quant.o")
    jobs.append(([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "qmv_quant.hip"), "-o", obj], obj))
    obj = os.path.join(BUILD, "qmv_scratch.o")
    jobs.append(([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "qmv_scratch.hip"), "-o", obj],
                 obj))
    obj = os.path.join(BUILD, "qmv_bench.o")
    jobs.append(([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "qmv_bench.hip"), "-o", obj], obj))
    obj = os.path.join(BUILD, "qmv_api.o")
    jobs.append((["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "qmv_api.cpp"), "-o", obj], obj))
    return jobs


def _run(cmd: list[str]) -> float:
    t0 = time.time()
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return time.time() - t0


def build(verbose: bool = False) -> str:
    """Compile everything and link libqmv.so. Always rebuilds. Returns the
    library path."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    t0 = time.time()
    jobs = _jobs()
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        futs = [ex.submit(_run, cmd) for cmd, _ in jobs]
        secs = [f.result() for f in futs]
    if verbose:
        for (cmd, obj), t in sorted(zip(jobs, secs), key=lambda js: -js[1]):
            print(f"  {t:6.1f} s  {os.path.basename(obj)}", flush=True)
    objs = [o for _, o in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f} s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
