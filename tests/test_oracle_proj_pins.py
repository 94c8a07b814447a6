"""The projection oracle against hand-worked values and closed forms (CPU only)."""
import pytest

import oracle
from oracle_proj_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_proj_pin(pin):
    pin(oracle.get_proj())
