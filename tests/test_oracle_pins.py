"""The CPU oracle against hand-worked cases, closed forms, invariants and brute force."""
import pytest

from tests.oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(orc, pin):
    pin(orc)
