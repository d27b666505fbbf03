import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.build()
    oracle.set_mutation(oracle.MUT_NONE)
    return oracle


@pytest.fixture
def mutated(orc):
    """Plant one oracle mistake for the duration of a test, then remove it."""
    planted = []

    def plant(m):
        orc.set_mutation(m)
        planted.append(m)

    yield plant
    orc.set_mutation(orc.MUT_NONE)
