"""The CPU oracle against its pins (pages' printed numbers, closed forms, library routines, brute force)."""
import pytest

from oracle import zha_oracle
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(zha_oracle)
