"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.load())
