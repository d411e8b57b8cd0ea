"""Build libpariskv.so (HIP, gfx950) in-tree with hipcc.

Usage: python kv_cache_top_amd/build.py   (or __graft_entry__.build()).
Run it as a script: importing the package loads the library it rebuilds.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpariskv.so")
BUILD_DIR = os.path.join(PKG, "_build")

HIP_SOURCES = ["pk_api.hip", "pk_encode.hip", "pk_scan.hip", "pk_retrieve.hip", "pk_attend.hip",
               "pk_fused.hip", "pk_kmeans.hip"]
CXX_SOURCES = ["pk_codebook.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: the integer path (ids, codes, votes) is defined by
# uncontracted fp32 arithmetic; kernels that want FMA call fmaf explicitly.
# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 are generated.
COMMON = ["-O3", "-fPIC", "-std=c++17", "-I", os.path.join(ROOT, "include")]
HIP_FLAGS = ["--offload-arch=gfx950", "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return r


def _check_no_scratch(src: str, remarks: str) -> None:
    """Every kernel must keep its state in registers and LDS: a private (scratch)
    segment means per-lane memory round trips inside the hot loops."""
    name = None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].split("[")[0].strip()
        elif "ScratchSize [bytes/lane]:" in line:
            size = int(line.split("ScratchSize [bytes/lane]:")[1].split("[")[0])
            if size != 0:
                raise RuntimeError(f"{src}: kernel {name} uses {size} B/lane of scratch")


def build(verbose: bool = False) -> str:
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append((obj, [HIPCC, "-x", "hip", *COMMON, *HIP_FLAGS,
                           "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src),
                           "-o", obj], src))
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append((obj, ["g++", *COMMON, "-Wall", "-c", os.path.join(CSRC, src), "-o", obj], None))

    def one(job):
        r = _run(job[1])
        if job[2] is not None:
            _check_no_scratch(job[2], r.stdout + r.stderr)
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1, 16)) as ex:
        list(ex.map(one, jobs))
    objs = [j[0] for j in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
