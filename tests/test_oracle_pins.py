"""The fp64 oracle against closed forms, special cases, brute force and
invariants (CPU only)."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.load())
