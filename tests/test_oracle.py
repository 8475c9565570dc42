"""The CPU oracle against its pins (hand-worked goldens, IEEE fp16, closed
forms, invariants, exact rational brute force).  CPU only."""
import pytest

from oracle import pnref
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(pnref.default())


def test_oracle_rejects_bad_shapes():
    o = pnref.default()
    import numpy as np
    with pytest.raises(ValueError):
        o.gemv_f64("pn3t", np.zeros(34, np.uint8), 1, 81, np.zeros(81, np.float16))
    with pytest.raises(ValueError):
        o.dequantize("pn4t", np.zeros(34, np.uint8), 1, 100)
