"""The CPU oracle against its pins (closed forms, hand counts, library
routines, brute force).  CPU only."""

import pytest

import oracle_pins

PINS = oracle_pins.ALL_PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin()
