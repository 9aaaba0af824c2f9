"""The CPU oracle against hand-worked values, closed forms, invariants, brute force and
PyTorch's own quantiser (no GPU needed)."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.loco_oracle)
