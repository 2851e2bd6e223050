import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")

# The host-sanitizer run (rank_gemm_svdq_amd/build.py --sanitize) points the
# binding at the instrumented library through SVDQ_TEST_LIB.
if os.environ.get("SVDQ_TEST_LIB"):
    import rank_gemm_svdq_amd.binding as _binding
    _binding.LIB_PATH = os.path.abspath(os.environ["SVDQ_TEST_LIB"])


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size CPU work (minutes)")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN
