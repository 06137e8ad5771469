"""The fp64 oracle agrees with every pin (closed forms, series, asymptotics,
limits, finite differences, rounding references).  CPU only."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)
