"""The float64 oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, lib):
    pin(lib)


def test_oracle_rejects_bad_shapes():
    import numpy as np

    with pytest.raises(ValueError):
        oracle.attn_fwd(np.zeros((1, 2, 3)), np.zeros((1, 2, 4)), np.zeros((1, 2, 4)), 1.0)
    with pytest.raises(RuntimeError):
        oracle.attn_fwd(np.zeros((1, 2, 3)), np.zeros((1, 0, 3)), np.zeros((1, 0, 3)), 1.0)
