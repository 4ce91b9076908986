"""The CPU oracle against its pins (library routines, closed forms, brute
force, the Gumbel-max theorem and the router example printed on P5 §3.1)."""
import pytest

from tests import oracle_pins

PINS = oracle_pins.ALL_PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(oracle, pin):
    pin(oracle)
