"""Build the C-ABI shared library in-tree (rank_gemm_svdq_amd/lib/libsvdq.so).

Host sources are compiled with g++ (x86-64-v3, no fp contraction in the
packers), device sources with hipcc for gfx950; hipcc links the library.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libsvdq.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HOST_FLAGS = ["-O3", "-march=x86-64-v3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function"]
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

UNITS = [
    ("host_prepare.cpp", ["g++"] + HOST_FLAGS + ["-ffp-contract=off"]),
    ("host_eigen.cpp", ["g++"] + HOST_FLAGS + ["-ffp-contract=fast"]),
    ("device_kernels.hip", [HIPCC] + DEVICE_FLAGS),
    ("device_search.hip", [HIPCC] + DEVICE_FLAGS),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return out


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    objs = []
    for src, cc in UNITS:
        obj = os.path.join(BUILD, src + ".o")
        out = _run(cc + ["-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out:
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + ["-lpthread"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
