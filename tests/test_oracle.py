"""CPU tests of the fp64 oracle: every pin passes on the real oracle, and every
planted mistake (a patched copy of the oracle source, tests/oracle_mutants.py)
fails at least one pin."""
import os

import numpy as np
import pytest

import oracle
from oracle_mutants import MUTANTS, mutant_source
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, mutant):
    src = tmp_path / ("oracle_m%d.c" % mutant)
    src.write_text(mutant_source(mutant))
    path = oracle.build(str(tmp_path / ("liboracle_m%d.so" % mutant)), source=str(src))
    bad = oracle.Oracle(path)
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(bad)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "planted mistake %d (%s) passed every pin" % (mutant, MUTANTS[mutant][0])


def test_rows_interface_matches_fwd(orc):
    """The per-row entry used for sampled checks agrees with the full forward."""
    rng = np.random.default_rng(5)
    B, H, L, d = 1, 1, 40, 8
    q, k, v, r = (rng.standard_normal((B, H, L, d)) for _ in range(4))
    o, lse = orc.fwd(q, k, v, r, window=7, n_sink=2)
    pos = np.array([0, 3, 17, 39])
    o2, lse2 = orc.rows(q[0, 0, pos], r[0, 0, pos], pos, k[0, 0], v[0, 0],
                        scale=1 / np.sqrt(d), window=7, n_sink=2)
    np.testing.assert_array_equal(o2, o[0, 0, pos])
    np.testing.assert_array_equal(lse2, lse[0, 0, pos])


def test_rejects_bad_arguments(orc):
    k = np.zeros((4, 2))
    with pytest.raises(ValueError):
        orc.rows(np.zeros((1, 2)), np.zeros((1, 2)), [4], k, k, scale=1.0)
    with pytest.raises(ValueError):
        orc.rows(np.zeros((1, 2)), np.zeros((1, 2)), [-2], k, k, scale=1.0)


def test_thread_count_does_not_change_result(orc):
    rng = np.random.default_rng(6)
    q, k, v, r = (rng.standard_normal((1, 2, 64, 16)) for _ in range(4))
    a = orc.fwd(q, k, v, r, nthreads=1)
    b = orc.fwd(q, k, v, r, nthreads=max(2, os.cpu_count() or 2))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_backward_thread_count(orc):
    """Backward: row gradients are exact per row; key and value gradients are
    sums whose order depends on the thread count only (fixed count: fixed result)."""
    rng = np.random.default_rng(7)
    q, k, v, r, do = (rng.standard_normal((1, 2, 64, 16)) for _ in range(5))
    a = orc.bwd(q, k, v, r, do, window=9, n_sink=2, nthreads=1)
    b = orc.bwd(q, k, v, r, do, window=9, n_sink=2, nthreads=3)
    c = orc.bwd(q, k, v, r, do, window=9, n_sink=2, nthreads=3)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[3], b[3])
    for x, y, z in zip(a, b, c):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(y, z)


def test_backward_rejects_bad_shapes(orc):
    x = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        orc.bwd(x, x, x, x, np.zeros((1, 1, 4, 3)))
