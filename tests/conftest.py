import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (oracle runs take tens of seconds)")


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding; fails loudly (never skips) when the GPU or library is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu-marked test run without a visible GPU (deselect with -m 'not gpu')")
    from lm_head_linear_tiled_amd import binding
    if os.environ.get("FLCE_LIB"):  # a measurement variant of the library (same sources, other build macros)
        binding.LIB_PATH = os.path.abspath(os.environ["FLCE_LIB"])
    binding.load()  # raises if libflce.so is missing
    return binding
