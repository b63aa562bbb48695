"""The CPU oracle against its pins (hand values, page figures, closed forms,
brute force).  No GPU."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
