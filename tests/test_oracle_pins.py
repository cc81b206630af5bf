"""The oracle checked against its pins (tests/pins.py); CPU only."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    assert orc.mutant() == 0
    pin(orc)
