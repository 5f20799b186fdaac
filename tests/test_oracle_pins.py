"""The fp64 oracle against its pins (library special cases, closed forms,
brute force, the hand-computed gate example and the pages' invariants).
See tests/oracle_pins.py for what each pin checks and why it is independent."""
import pytest

import oracle.seer_oracle as O
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(O)
