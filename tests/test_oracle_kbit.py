"""The k-bit quantized GEMV part of the CPU oracle against its pins (CPU only)."""
import pytest

import oracle_kbit_pins as P


@pytest.mark.parametrize("pin", P.ALL_KBIT_PINS, ids=lambda p: p.__name__)
def test_kbit_pin(oracle_lib, pin):
    pin(oracle_lib)
