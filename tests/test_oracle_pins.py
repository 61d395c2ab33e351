"""The CPU oracle against its pins (library routines, closed forms,
invariants); see tests/oracle_pins.py for what each pin fixes."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.get())
