"""The oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle_pins as pins
from oracle import eplb_oracle as o


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(o)
