"""The CPU oracle against closed forms, brute force, identities and
hand-derived values (no GPU)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
