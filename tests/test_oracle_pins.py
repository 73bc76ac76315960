"""The oracle against its pins (exact arithmetic, brute force, closed forms,
worked examples, library routines).  CPU only."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=[p.__name__ for p in pins.ALL_PINS])
def test_pin(pin):
    pin()
