"""The oracle against its pins: library special cases, closed forms, invariants,
brute force and the worked examples under tests/golden (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=[p.__name__ for p in pins.ALL_PINS])
def test_pin(pin, orc):
    pin(orc)
