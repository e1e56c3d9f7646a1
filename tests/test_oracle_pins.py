"""The fp64 oracle against its pins (closed forms, special cases, causality,
associativity, FAVOR+ unbiasedness and convergence, finite differences)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()
