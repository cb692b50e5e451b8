"""The CPU oracle against its pins (closed forms, invariants, brute force and
library special cases)."""
import pytest

from oracle import dflash_oracle
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(dflash_oracle)
