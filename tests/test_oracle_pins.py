"""The oracle against closed forms, brute force, dense attention and invariants (CPU)."""
import pytest

import oracle.spin_oracle as om
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(om)
