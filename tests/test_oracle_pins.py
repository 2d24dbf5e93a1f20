"""The oracle against its pins (library routines, closed forms, brute force)."""
import pytest

from oracle import star_oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(star_oracle)
