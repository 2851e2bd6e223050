"""The host half of the library (preparation, eigen-solver, packers, layout
conversions, argument checks) under AddressSanitizer and
UndefinedBehaviorSanitizer: the host sources are rebuilt instrumented
(rank_gemm_svdq_amd/build.py, sanitize=True) and the host-library tests run
against that build in a subprocess with the sanitizer runtimes preloaded.
Any memory error or undefined behaviour aborts the subprocess."""
import os
import shutil
import subprocess
import sys

import pytest

from rank_gemm_svdq_amd import build as BLD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++ with the sanitizer runtimes")
def test_host_library_is_clean_under_asan_and_ubsan():
    lib = BLD.build(sanitize=True, reuse_device_objects=True)
    env = dict(os.environ)
    env.update(BLD.sanitizer_env())
    env["SVDQ_TEST_LIB"] = lib
    env.pop("PYTEST_XDIST_WORKER", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:xdist", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_host_library.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=1200)
    tail = r.stdout[-3000:]
    assert r.returncode == 0, tail
    assert " passed" in tail and " failed" not in tail, tail
    assert "AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout, tail
