"""The fp64 oracle against what the pages and mathematics fix (CPU only)."""
import pytest

import oracle
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


def test_mla_dims_and_scale():
    P.pin_mla_dims_and_scale()
