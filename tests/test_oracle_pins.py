"""The CPU oracle against its pins (no GPU)."""

import pytest

import oracle.dense_fp64 as ob
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(ob)
