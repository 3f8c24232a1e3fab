"""The fp64 oracle against what the GSI summary and mathematics fix (CPU only)."""
import pytest

from oracle import gsi_oracle as orc
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(orc)
