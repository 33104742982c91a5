"""The oracle against its pins (worked examples, closed forms, library
routines, brute force, Blelloch, invariants).  CPU only."""
import pytest

from pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(orc, pin):
    pin(orc)
