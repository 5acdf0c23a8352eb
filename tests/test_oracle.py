"""The CPU oracle against its pins (no GPU)."""
import pytest

from oracle import liftquant_ref, refpack
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(liftquant_ref, refpack)
