"""The CPU oracle against its pins (brute force, closed forms, invariants, library routines)."""
import pytest

import oracle
from tests import oracle_pins

pytestmark = pytest.mark.cpu


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS + oracle_pins.FFN_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)
