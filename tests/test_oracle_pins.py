"""The fp64 oracle against its pins (closed forms, brute force, invariants, worked examples)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(o, pin):
    pin(o)
