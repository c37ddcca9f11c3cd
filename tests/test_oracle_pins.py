"""The oracle against its pins (CPU)."""

import pytest

import oracle
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("name", sorted(ALL_PINS))
def test_pin(name):
    ALL_PINS[name](oracle)
