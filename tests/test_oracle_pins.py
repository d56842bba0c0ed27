"""CPU: the oracle against its pins (closed forms, invariants, brute force,
exact arithmetic, library routines and the pages' printed geometry)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)
