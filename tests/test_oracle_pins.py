"""The CPU oracle against its pins (brute force, closed forms, dense Gated DeltaNet)."""
import pytest

import oracle.sdm_oracle as O
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(O)
