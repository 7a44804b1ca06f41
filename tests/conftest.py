import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload, minutes")


@pytest.fixture(scope="session")
def oracle():
    from oracle import build, lco
    if not os.path.exists(lco.LIB_PATH):
        build.build()
    lco.lib()
    return lco


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    """A cited fixture from tests/golden/ (values worked by hand from the
    pages' definitions, stated on the pages, or published with a method the
    code uses; never produced by the library)."""
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)
