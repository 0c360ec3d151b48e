"""The fp64 oracle against closed forms, invariants and library routines."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_decode_is_one_token_recurrence(orc):
    """decode() is the packed recurrence with one token per sequence."""
    import numpy as np
    r = np.random.default_rng(3)
    N, H, HV, dk, dv = 3, 2, 4, 8, 8
    q = r.standard_normal((N, H, dk)).astype(np.float32)
    k = r.standard_normal((N, H, dk)).astype(np.float32)
    v = r.standard_normal((N, HV, dv)).astype(np.float32)
    g = -r.random((N, HV)).astype(np.float32)
    b = r.random((N, HV)).astype(np.float32)
    s = r.standard_normal((N, HV, dv, dk))
    o1, s1 = orc.decode(q, k, v, g, b, s)
    for n in range(N):
        on, sn = orc.recurrence(q[n:n + 1], k[n:n + 1], v[n:n + 1], g[n:n + 1], b[n:n + 1],
                                np.array([0, 1]), s0=s[n:n + 1])
        assert np.array_equal(on[0], o1[n]) and np.array_equal(sn[0], s1[n])
