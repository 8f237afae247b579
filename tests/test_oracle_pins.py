"""The fp64 oracle against facts the pages and mathematics fix (CPU only)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
