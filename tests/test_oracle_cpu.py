"""The CPU oracle against its pins (textbook routines, closed forms,
invariants, hand-worked fixtures, brute force).  No GPU needed."""
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=[p.__name__ for p in pins.ALL_PINS])
def test_oracle_pin(oracle, pin):
    pin(oracle)
