"""The KV4 decode-attention oracle against its pins (CPU only)."""
import pytest

import oracle
from kv4_pins import KV4_PINS


@pytest.mark.parametrize("pin", KV4_PINS, ids=[p.__name__ for p in KV4_PINS])
def test_kv4_oracle_pin(pin):
    pin(oracle)
