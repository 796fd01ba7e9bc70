"""Build libtq.so (HIP kernels for gfx950 + host C ABI) in-tree.

    python compressed_domain_decode_amd/build.py

The kernels are compiled with hipcc for gfx950 only. Packed-fp32 VALU
instructions are disabled (-packed-fp32-ops); host code is plain g++.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtq.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
              f"-I{ROCM}/include"]

HIP_SOURCES = ["encode.hip", "attend.hip", "probe.hip", "cache.hip", "dense.hip", "scratch.hip"]
HOST_SOURCES = ["codec.cpp", "api.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {os.path.basename(cmd[-1])}")
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, "-c", "-o", obj, os.path.join(CSRC, src)])
    for src in HOST_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        jobs.append(["g++", *HOST_FLAGS, "-c", "-o", obj, os.path.join(CSRC, src)])
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(_run, jobs))
    objs = [os.path.join(OUT_DIR, s + ".o") for s in HIP_SOURCES + HOST_SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
          "-Wl,--exclude-libs,ALL", "-lquadmath"])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
