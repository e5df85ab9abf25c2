import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")

# A test build of the library (the host-sanitizer test runs test_abi.py against one).
if os.environ.get("WQ_TEST_LIB"):
    import gemv_wq_gemm_amd
    gemv_wq_gemm_amd.LIB_PATH = os.environ["WQ_TEST_LIB"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def golden_path(name: str) -> str:
    return os.path.join(GOLDEN, name)


@pytest.fixture(scope="session")
def gpu_device():
    """cuda:0, or skip when no GPU is present."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")
