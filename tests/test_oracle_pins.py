"""The CPU oracle against its pins (see oracle_pins.py for what each pins)."""
import pytest

from oracle import oracle as O
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return O.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, lib):
    pin(lib)
