"""The oracle against its pins (CPU only)."""
import pytest

import oracle_pins
from oracle import dms_oracle


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(dms_oracle)
