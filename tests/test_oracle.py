"""The CPU oracle against its pins (closed forms, library routines, invariants)."""
import pytest

import oracle_pins as P


@pytest.fixture(scope="module")
def real_oracle():
    from oracle import build
    build.build()
    return P.OracleUnderTest()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, real_oracle):
    pin(real_oracle)


def test_threads_do_not_change_bits(real_oracle):
    """Each output row is summed serially, so the OpenMP thread count cannot change a bit."""
    import numpy as np
    wl = P.tiny(1200, B=4, QH=8, KVH=2, D=16, ps=4)
    a = real_oracle.attend(wl, nthreads=1)
    b = real_oracle.attend(wl, nthreads=4)
    assert np.array_equal(a, b)


def test_row_subset_matches_full(real_oracle):
    import numpy as np
    wl = P.tiny(1300, B=3, QH=8, KVH=4, D=8, ps=4)
    full = real_oracle.attend(wl)
    rows = [0, 5, 9, 23, 17]
    sub = real_oracle.attend(wl, rows=rows)
    assert np.array_equal(sub, full.reshape(-1, wl.head_dim)[rows])
