"""CPU tests: the fp64 oracle against its pins (see tests/oracle_pins.py)."""

import pytest

from oracle import online, ref
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(ref, online)
