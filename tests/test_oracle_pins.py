"""The CPU oracle against its pins (see oracle_pins.py for what each rests on)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle)
