"""The CPU oracle against its pins (exact arithmetic, enumeration, closed
forms, library special cases, stated invariants, metamorphic relations)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(o, pin):
    pin(o)


def test_rejects_bad_configs(o):
    import numpy as np
    L = np.zeros((1, 16))
    b = np.zeros(16, np.float32)
    for (G, KG, K) in [(3, 1, 2), (4, 5, 2), (16, 2, 1), (4, 1, 5), (0, 1, 1), (4, 2, 0)]:
        with pytest.raises(ValueError):
            o.select(L, b, G, KG, K, 1.0)
    with pytest.raises(ValueError):
        o.dispatch(np.array([[0, 16]], np.int32), 16)
