"""The fp64 calibration oracle against what the GSI summary and mathematics fix (CPU only)."""
import pytest

from oracle import gsi_calibration as cal
from tests import calibration_pins


@pytest.mark.parametrize("pin", calibration_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(cal)
