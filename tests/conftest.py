import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    # a different build of the library (the host-sanitized one) for host tests
    alt = os.environ.get("MXQ_TEST_LIB")
    if alt:
        import mx_bit_quantized_amd as mxq
        mxq.LIB_PATH = alt
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def golden_path(name):
    return os.path.join(GOLDEN, name)


def golden_lines(name):
    with open(golden_path(name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()
