"""The CPU oracle against its pins (see tests/pins.py for what pins what)."""
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda p: p.__name__)
def test_pin(o, pin):
    pin(o)


def test_bound_formula():
    # |err| <= 1e-5 * sum_k |A x| + 1e-6, element-wise.
    import numpy as np
    b = oracle.bound(np.array([0.0, 1.0, 2.5e5]))
    assert np.allclose(b, [1e-6, 1e-5 + 1e-6, 2.5 + 1e-6], rtol=0, atol=1e-15)


def test_pad_model():
    import numpy as np
    f = oracle.pad_after_reset(3, 40, 0b101)
    assert f.shape == (3, 10)  # ceil(40 / 4) flag tiles
    assert (f[0] == 0xFFFFFFFF).all() and (f[1] == 0).all() and (f[2] == 0xFFFFFFFF).all()
    g = oracle.pad_after_calls(f, 1, 5)
    assert (g[1] == 5).all() and np.array_equal(g[[0, 2]], f[[0, 2]])
    tiles, first = oracle.expected_timeouts(g, 1)
    assert tiles == [] and first is None
    h = g.copy()
    h[2, 1] = 3
    tiles, first = oracle.expected_timeouts(h, 1)
    assert tiles == [1] and first == (1, 2)
    tiles, first = oracle.expected_timeouts(oracle.pad_after_reset(4, 33, 0b0001), 1)
    assert tiles == list(range(9)) and first == (0, 2)
