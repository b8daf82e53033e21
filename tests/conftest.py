import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(autouse=True)
def _automatic_kernel_choice():
    """Every test starts and ends with the library's automatic kernel choice
    (the kernel-choice overrides are process-wide)."""
    from mixture_value_projection_amd import binding
    yield
    if binding._LIB is not None:
        binding.clear_overrides()
