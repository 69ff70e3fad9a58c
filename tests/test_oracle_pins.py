"""The fp64 oracle against facts that do not come from it (CPU only)."""

import pytest

import oracle
from oracle_pins import PINS


@pytest.mark.parametrize("name", sorted(PINS))
def test_oracle_pin(name):
    pin, bound = PINS[name]
    err = pin(oracle)
    assert err <= bound, f"pin {name}: worst relative error {err:.3e} > {bound:.1e}"
