"""The oracle against its pins (CPU only)."""
import pytest

import _pins


@pytest.mark.parametrize("pin", _pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
