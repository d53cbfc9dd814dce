"""The oracle against hand values, closed forms and an independent formulation."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)
