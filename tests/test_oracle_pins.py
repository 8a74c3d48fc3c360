"""The CPU oracle against what the pages and mathematics fix (no GPU)."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.gqe_oracle)
