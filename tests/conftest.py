import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a 'key: values' fixture under tests/golden (lines starting with # are comments)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            out[key.strip()] = val.split()
    return out


@pytest.fixture(scope="session")
def i8l():
    """The binding, with libint8lin.so built in-tree first if it is missing."""
    import mixed_precision_quantized_int8_amd as pkg
    from mixed_precision_quantized_int8_amd import _binding, build

    if not os.path.exists(_binding.LIB_PATH):
        build.build_library()
    pkg.lib()
    return pkg
