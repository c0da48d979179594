"""The fp64 oracle against closed forms, library routines, invariants and
brute force (see tests/oracle_pins.py for what each pin fixes)."""
import pytest

import oracle
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(oracle.lra_oracle)
