import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size oracle runs (seconds to a minute on the CPU)")


# A test process may load another build of the library (the host-sanitized one, see
# tests/test_host_sanitized.py) instead of sparse_mixture_experts_02_amd/libmoe.so.
if os.environ.get("MOE_TEST_LIBRARY"):
    from sparse_mixture_experts_02_amd import binding as _binding
    _binding._LIB_PATH = os.environ["MOE_TEST_LIBRARY"]
