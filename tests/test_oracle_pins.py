"""The fp64 oracle against what the pages and mathematics fix (CPU only)."""

import pytest

from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()
