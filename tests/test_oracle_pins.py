"""The CPU oracle against its pins (format definition, a library cast, exact
arithmetic, hand-derived values and the method's invariants)."""

import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(quick=False)


def test_oracle_rejects_non_finite():
    """Non-finite input is outside the contract; the oracle refuses it."""
    import numpy as np
    import pytest

    import oracle

    for bits in (0x7FC0, 0x7F80, 0xFF80):          # NaN, +Inf, -Inf
        x = np.zeros((4, 4), dtype=np.uint16)
        x[1, 2] = bits
        with pytest.raises(ValueError):
            oracle.quantize(x, 2, 2)
        with pytest.raises(ValueError):
            oracle.tile_amax(x, 2, 2)
    with pytest.raises(ValueError):
        oracle.encode(float("nan"))
    with pytest.raises(ValueError):
        oracle.encode(449.0)
