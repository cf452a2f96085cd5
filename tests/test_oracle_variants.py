"""The comparison-GEMM oracle against its pins (no GPU)."""
import pytest

import oracle
from variant_pins import VARIANT_PINS


@pytest.mark.parametrize("pin", VARIANT_PINS, ids=[p.__name__ for p in VARIANT_PINS])
def test_variant_pin(pin):
    pin(oracle)
