"""The gradient oracle against finite differences of the forward and closed forms (CPU only)."""
import pytest

import oracle
from oracle_grad_pins import ADDRESS_PINS, SCAN_PINS


@pytest.fixture(scope="module")
def g():
    return oracle.get_grad()


@pytest.mark.parametrize("pin", SCAN_PINS, ids=lambda p: p.__name__)
def test_scan_grad_pin(g, pin):
    pin(g)


@pytest.mark.parametrize("pin", ADDRESS_PINS, ids=lambda p: p.__name__)
def test_address_grad_pin(g, pin):
    pin(g, oracle.get())
