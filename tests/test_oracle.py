"""The fp64 oracle against its pins (closed forms, brute force, a library
special case, invariants).  CPU only."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


import oracle_pins_fp8


@pytest.mark.parametrize("pin", oracle_pins_fp8.ALL_PINS, ids=lambda f: f.__name__)
def test_fp8_pin(pin):
    pin()
