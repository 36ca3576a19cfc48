"""The CPU oracle against its pins (closed forms, hand-derived fixtures, invariants)."""

import pytest

import pins


@pytest.mark.parametrize("pin", pins.PINS, ids=[p.__name__ for p in pins.PINS])
def test_pin(orc, pin):
    pin(orc)
