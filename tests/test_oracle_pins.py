"""The CPU oracle against its pins (hand traces, dense reduction, exact top-k,
closed forms and invariants).  CPU only."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.load())
