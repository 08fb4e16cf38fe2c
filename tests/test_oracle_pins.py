"""The CPU oracle against its pins (hand-worked values, closed forms, brute
force, invariants).  See oracle_pins.py for what each pin fixes."""
import pytest

from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
