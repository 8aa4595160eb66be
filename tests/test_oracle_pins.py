"""The CPU oracle against its pins (exact rationals, closed forms, library
routines in fp64, invariants, hand-derived examples)."""
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
