"""The CPU oracle against brute force, closed forms, library routines and
invariants (see tests/oracle_pins.py for what each pin checks)."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()
