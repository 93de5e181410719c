import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")

# The host-sanitizer test reruns CPU suites in a child process against the
# sanitizer-instrumented build of the library; it names that build here.
if os.environ.get("MOE_TEST_LIBRARY"):
    from mxfp4_routed_expert_renorm_amd import binding as _binding
    _binding.LIB_PATH = os.environ["MOE_TEST_LIBRARY"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def read_golden(name):
    """Rows of a whitespace-separated golden fixture, comments dropped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library, on a machine with a GPU; fails loudly otherwise."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test selected but no GPU is visible")
    from mxfp4_routed_expert_renorm_amd import lib
    return lib
