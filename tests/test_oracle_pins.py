"""The CPU oracle against its pins (format definition, a library cast, exact
arithmetic, hand-derived values and the method's invariants)."""

import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(quick=False)
