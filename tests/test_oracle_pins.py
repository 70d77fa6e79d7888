"""The oracle against its pins (hand-worked values, finite differences, library
routines, closed forms, invariants).  CPU only."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)
