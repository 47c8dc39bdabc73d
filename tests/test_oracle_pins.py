"""The CPU oracle against brute force, closed forms, invariants, hand-derived
golden values and independent library routines (CPU only)."""
import pytest

from oracle import egm_oracle
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(egm_oracle)
