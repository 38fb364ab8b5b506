import os

import pytest
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU check")


@pytest.fixture
def launch_override():
    """Set a launch-shape override (qlin_set_launch_override) for one test;
    every family it touched is restored to the library's own choice after."""
    from group_wise_bit_amd import qlin
    touched = set()

    def set_(family, cfg):
        touched.add(family)
        qlin.set_launch_override(family, cfg)
    yield set_
    for fam in touched:
        qlin.set_launch_override(fam, None)
