"""The oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(lib, pin):
    pin(lib)
