import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    oracle.lib()
    return oracle


@pytest.fixture
def force_table():
    """Setter for the library's decode-table test hook; the library's own
    choice is restored when the test ends."""
    import trellis_coded_bit_prefill_amd as tp

    yield tp.force_table
    tp.force_table(None)

