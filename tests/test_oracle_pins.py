"""The fp64 oracle against its pins: the worked example of "Lendo uma Projeção", brute force,
a library special case, closed forms and invariants. CPU only."""

import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)
