"""The CPU oracle against its pins (hand codes, an independent encoder, torch's
cast, closed-form tile and layout invariants).  No GPU."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
