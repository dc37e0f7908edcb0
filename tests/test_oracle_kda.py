"""The KDA chain-verify oracle (oracle/kda.c) against its pins (CPU only)."""
import pytest

import oracle
import oracle_kda_pins as P


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", P.ALL_KDA_PINS, ids=lambda p: p.__name__)
def test_kda_pin(orc, pin):
    pin(orc)
