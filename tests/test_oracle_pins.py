"""The CPU oracle against its pins (closed forms, invariants, golden values, brute force)."""
import pytest

from oracle import saf_oracle
from tests.oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(saf_oracle)
