"""The fp64 oracle against its pins (closed forms, invariants, library
routines, dense brute force).  See tests/oracle_pins.py for what each fixes."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)
