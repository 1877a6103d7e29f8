"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle as O
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)
