import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN


@pytest.fixture
def tune():
    """Sets launch-plan overrides (kvq_set_tuning) for one test and gives
    every knob back to the plan afterwards: tune("pages_per_wave", 3),
    tune("split_shape", "2x1s1"); None hands a knob back to the plan."""
    import fp8_kv_cache_write_amd as kv
    kv.reset_tuning()
    yield kv.set_tuning
    kv.reset_tuning()
