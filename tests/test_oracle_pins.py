"""The fp64 oracle against brute force, torch SDPA special cases, closed
forms, invariants and hand-worked golden cases (CPU only)."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()
