"""The FP64 oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.default())


def test_thread_count_does_not_change_result():
    import numpy as np
    rng = np.random.default_rng(30)
    q, k, v = (rng.standard_normal((2, 3, 33, 16)) for _ in range(3))
    o1, l1 = oracle.attention(q, k, v, causal=True, nthreads=1)
    o4, l4 = oracle.attention(q, k, v, causal=True, nthreads=4)
    assert np.array_equal(o1, o4) and np.array_equal(l1, l4)
