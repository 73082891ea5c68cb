"""The oracle against its pins (closed forms, brute force, invariants); CPU only."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle._load())
