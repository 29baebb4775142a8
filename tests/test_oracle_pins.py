"""The CPU oracle against its pins (see oracle_pins.py for what pins what)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)
