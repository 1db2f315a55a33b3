"""The fp64 oracle against closed forms, invariants, torch's cross-entropy,
finite differences and brute force (CPU only)."""
import pytest

from oracle import flce_oracle as O
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)
