"""The CPU oracle against its pins (format definition, closed forms, torch
routines, invariants). CPU only."""
import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()
