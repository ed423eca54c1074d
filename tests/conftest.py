import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly if run without a GPU; they are selected with -m gpu.
    pass


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    oracle.build()
    return oracle


def read_golden(name):
    path = os.path.join(ROOT, "tests", "golden", name)
    rows = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            rows[key] = vals
    return rows


def f16_copy_expected(bits):
    """What the packed activations' fp16 copy holds for bf16 values `bits`
    (uint16): the value times 2^8 as fp16 where that is exact, else the NaN
    marker 0x7FFF (the library's packed-activation layout)."""
    import numpy as np

    a = (bits.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        h = (a * np.float32(256)).astype(np.float16)
        exact = h.astype(np.float32) / np.float32(256) == a
    return np.where(exact, h.view(np.uint16), np.uint16(0x7FFF)).astype(np.uint16)
