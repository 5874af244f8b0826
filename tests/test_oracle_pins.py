"""The CPU oracle against what the pages and mathematics fix (no GPU)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load_library()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, lib):
    pin(lib)


def test_thread_count_does_not_change_results(lib):
    import numpy as np
    rng = np.random.default_rng(3)
    p = oracle_pins._rand_problem(rng, 3, 64, 17, 16)
    y1, h1 = oracle.scan(nthreads=1, lib=lib, **p)
    y8, h8 = oracle.scan(nthreads=8, lib=lib, **p)
    assert np.array_equal(y1, y8) and np.array_equal(h1, h8)


def test_zoh_entry_point(lib):
    import math
    abar, c = oracle.zoh(0.1, -2.0)
    assert abar == math.exp(-0.2) and abs(c - (math.exp(-0.2) - 1) / -2.0) < 1e-16
    assert oracle.zoh(0.25, 0.0) == (1.0, 0.25)


def test_backward_thread_count_changes_only_rounding(lib):
    import numpy as np
    rng = np.random.default_rng(4)
    p = oracle_pins._rand_problem(rng, 2, 40, 19, 16)
    dy = rng.standard_normal(p["x"].shape)
    g1 = oracle.scan_bwd(nthreads=1, lib=lib, dy=dy, **p)
    g8 = oracle.scan_bwd(nthreads=8, lib=lib, dy=dy, **p)
    for k in ("dx", "ddelta", "dz", "dA", "dD", "dh0"):     # per channel: identical
        assert np.array_equal(g1[k], g8[k]), k
    for k in ("dB", "dC"):                                   # channel sums: rounding only
        assert np.max(np.abs(g1[k] - g8[k])) <= 1e-13 * np.max(np.abs(g1[k]))
