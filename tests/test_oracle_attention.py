"""Oracle attention and cache-model pins (CPU only).  Each check is described
in tests/oracle_pins.py together with what fixes its expectation."""
import pytest

import oracle
import oracle_pins  # noqa: E402


@pytest.mark.parametrize("name", sorted(oracle_pins.ALL_CHECKS))
def test_pin(name):
    oracle_pins.ALL_CHECKS[name](oracle.load())


def test_ring_refuses_an_append_that_drops_visible_rows():
    import numpy as np
    from oracle.cache_model import OracleCache, RangeError
    c = OracleCache(1, 1, 32, 16, window=8, ring_step=4)
    x = np.zeros((1, 14, 1, 32), np.float32)
    c.append(x, x)
    with pytest.raises(RangeError):          # 14 + 9 rows: base 8 > 14 + 1 - 8
        c.append(np.zeros((1, 9, 1, 32), np.float32), np.zeros((1, 9, 1, 32), np.float32))
    assert c.len[0] == 14 and c.base[0] == 0  # refused before any change


def test_rebase_schedule_of_the_sink_ring_shape():
    """2048-row ring, 512-row step, window 1024, one row per append: the base
    advances by 512 every 512 appends once 2048 rows exist; at absolute length
    131072 the base is 129024 and the live window is physical rows [1024, 2048)."""
    import numpy as np
    from oracle.cache_model import OracleCache
    c = OracleCache(1, 1, 32, 2048, window=1024, ring_step=512)
    bases = {}
    for L in list(range(2040, 2600)) + [131071]:
        c.len[0] = L
        bases[L] = c.plan_base(0, 1)
        c.base[0] = bases[L]
    assert bases[2047] == 0 and bases[2048] == 512 and bases[2559] == 512 and bases[2560] == 1024
    assert bases[131071] == 129024
    L = 131072
    assert (max(0, L - 1024) - bases[131071], L - bases[131071]) == (1024, 2048)


def test_flat_cache_refuses_past_capacity():
    import numpy as np
    from oracle.cache_model import OracleCache, CapacityError
    c = OracleCache(2, 1, 32, 10)
    x = np.zeros((2, 8, 1, 32), np.float32)
    c.append(x, x)
    with pytest.raises(CapacityError):
        c.append(np.zeros((2, 3, 1, 32), np.float32), np.zeros((2, 3, 1, 32), np.float32))
    c.append(np.zeros((2, 3, 1, 32), np.float32), np.zeros((2, 3, 1, 32), np.float32), counts=[2, 0])
    assert list(c.len) == [10, 8]
