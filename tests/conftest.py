import json
import math
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)

GOLDEN = os.path.join(TESTS, "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large shapes (still minutes at most)")


def golden_value(v):
    """Fixture scalars: numbers, or the strings "-inf", "inf", "nan", "-0.0"."""
    if isinstance(v, str):
        return {"-inf": -math.inf, "inf": math.inf, "nan": math.nan,
                "-0.0": -0.0}[v]
    return float(v)


def golden_array(x, dtype=np.float64):
    def conv(y):
        if isinstance(y, list):
            return [conv(z) for z in y]
        return golden_value(y)
    return np.array(conv(x), dtype=dtype)


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.load()
