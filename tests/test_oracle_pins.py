"""The oracle against library routines, closed forms and invariants (CPU only)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("name", sorted(oracle_pins.ALL_PINS))
def test_pin(name):
    oracle_pins.ALL_PINS[name](None)
