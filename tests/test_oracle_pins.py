"""The fp64 oracle against its pins (closed forms, invariants, library routines, brute force)."""
import pytest

import oracle
from oracle_pins import ALL_PINS, bound_oracle


@pytest.fixture(scope="module")
def ora():
    return bound_oracle(oracle.load())


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(ora, pin):
    pin(ora)
