"""Run the CPU test suite against AddressSanitizer + UndefinedBehaviorSanitizer
builds of the host code: the C ABI layer (api.cpp), the codec set-up
(codec.cpp) and the C oracle (tq_oracle.c).

    python tests/run_sanitized.py [extra pytest args]

The GPU kernels are linked in unchanged from the regular build (sanitizers
apply to host code only); the package and the oracle load the sanitized
libraries through TQ_LIB_PATH / TQ_ORACLE_LIB, with libasan preloaded into the
Python process. Any sanitizer report aborts the run (halt_on_error)."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "compressed_domain_decode_amd")
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(ROOT, "tests", "_build", "san")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def sh(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def main(argv):
    os.makedirs(OUT, exist_ok=True)
    # the kernels and their launchers: the regular build's objects
    sys.path.insert(0, PKG)
    import build as tqbuild  # noqa: E402  (compressed_domain_decode_amd/build.py)
    tqbuild.build()
    hip_objs = [os.path.join(tqbuild.OUT_DIR, s + ".o") for s in tqbuild.HIP_SOURCES]
    host_objs = []
    for src in tqbuild.HOST_SOURCES:
        obj = os.path.join(OUT, src + ".o")
        sh(["g++", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
            *SAN, "-c", "-o", obj, os.path.join(CSRC, src)])
        host_objs.append(obj)
    lib = os.path.join(OUT, "libtq_san.so")
    sh(["g++", "-shared", *SAN, "-o", lib, *host_objs, *hip_objs, f"-L{ROCM}/lib",
        "-lamdhip64", "-lquadmath", f"-Wl,-rpath,{ROCM}/lib"])
    olib = os.path.join(OUT, "_tq_oracle_san.so")
    sh(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", *SAN,
        "-o", olib, os.path.join(ROOT, "oracle", "tq_oracle.c"), "-lm"])
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    ubsan = subprocess.check_output(["gcc", "-print-file-name=libubsan.so"], text=True).strip()
    env = dict(os.environ)
    env.update(
        TQ_LIB_PATH=lib, TQ_ORACLE_LIB=olib,
        LD_PRELOAD=" ".join([asan, ubsan] + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else [])),
        # Python and torch keep allocations until exit: leaks are not this code's
        ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
        UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-x", "-q", "-m",
           "not gpu", "-p", "no:cacheprovider", *argv]
    print("+", " ".join(cmd), flush=True)
    return subprocess.call(cmd, env=env, cwd=ROOT)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
