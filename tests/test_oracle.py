"""The CPU oracle against facts outside itself (library routines, closed forms, invariances,
brute force and the layout properties the header promises). CPU only."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(oracle)
