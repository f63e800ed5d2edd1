"""The oracle against its pins (closed forms, identities, exact brute force, worked cases)."""
import pytest

import oracle.verify_ref as ref
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(ref)
