"""The CPU oracle against its pins (see tests/oracle_pins.py).  CPU only."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("name", sorted(oracle_pins.PINS))
def test_pin(orc, name):
    oracle_pins.PINS[name](orc)


def test_oracle_has_no_planted_mistake(orc):
    assert orc.mutant() == 0
