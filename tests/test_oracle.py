"""The CPU oracle against closed forms, invariants, scipy, brute force and a hand-derived
fixture (see ``oracle_pins.py``).  CPU only."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
