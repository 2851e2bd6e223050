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
    ("device_probe.hip", [HIPCC] + DEVICE_FLAGS),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return out


# Host-code sanitizer configuration (CPU testing only): the host units with
# AddressSanitizer and UndefinedBehaviorSanitizer (g++), the device units as
# usual, linked by g++ into a separate library.  Python is not instrumented,
# so a process that loads it preloads the sanitizer runtimes (see
# sanitizer_env()).
ASAN_LIB = os.path.join(HERE, "lib_asan", "libsvdq.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def sanitizer_env():
    """Environment for a process that loads the sanitized library."""
    rt = [subprocess.run(["g++", f"-print-file-name={n}"], stdout=subprocess.PIPE, text=True).stdout.strip()
          for n in ("libasan.so", "libubsan.so")]
    return {"LD_PRELOAD": ":".join(rt), "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
            "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def build(verbose=False, sanitize=False, reuse_device_objects=False):
    """Compile and link the library.  sanitize: the host-sanitizer
    configuration above; reuse_device_objects (with sanitize): take the
    device objects of the last plain build instead of compiling them again."""
    bdir = BUILD + ("_asan" if sanitize else "")
    lib = ASAN_LIB if sanitize else LIB
    os.makedirs(bdir, exist_ok=True)
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    objs = []
    for src, cc in UNITS:
        if sanitize and reuse_device_objects and cc[0] != "g++":
            prev = os.path.join(BUILD, src + ".o")
            if os.path.exists(prev):
                objs.append(prev)
                continue
        obj = os.path.join(bdir, src + ".o")
        flags = cc + (SANITIZE_FLAGS if sanitize and cc[0] == "g++" else [])
        out = _run(flags + ["-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out:
            print(out)
        objs.append(obj)
    tmp = lib + ".tmp"
    if sanitize:
        _run(["g++", "-shared", "-fPIC"] + SANITIZE_FLAGS + ["-o", tmp] + objs +
             ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lpthread"])
    else:
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + ["-lpthread"])
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
