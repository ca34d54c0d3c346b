"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)
