"""Pins for the oracle's vertical-line selection (CPU only)."""

import itertools

import numpy as np
import pytest

from oracle import select


def _brute_topk(mass, k):
    """Best k-subset by total mass; among equals the lexicographically
    smallest index tuple (the lower-index tie rule)."""
    best = None
    for comb in itertools.combinations(range(len(mass)), k):
        key = (-sum(mass[list(comb)]), comb)
        if best is None or key < best:
            best = key
    return np.array(best[1], dtype=np.int64) if best else np.zeros(0, np.int64)


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = 9
    mass = rng.integers(0, 4, size=n + 3).astype(np.float64)   # many exact ties
    for window in (0, 1, 3):
        ctx = n + 3 - (3 - window)
        for num, den in ((1, 3), (1, 2), (5, 100), (1, 1)):
            k, cand = select.n_select(ctx, window, num, den)
            got = select.topk_vertical(mass, ctx, window, num, den)
            np.testing.assert_array_equal(got, _brute_topk(mass[:cand], k))


def test_select_count_is_integer_ceil():
    assert select.n_select(32768, 128, 5, 100) == (1632, 32640)
    assert select.n_select(128, 128, 5, 100) == (0, 0)
    assert select.n_select(100, 0, 5, 100) == (5, 100)
    assert select.n_select(101, 0, 5, 100) == (6, 101)


def test_colmass_total_mass_invariant():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((200, 64))
    q = rng.standard_normal((12, 64)) * 3
    cm0 = rng.uniform(0, 1, size=256)
    cm = select.colmass_update(cm0, q, k, 150)
    np.testing.assert_allclose(cm.sum() - cm0.sum(), 12.0, atol=1e-12)
    assert (cm[150:] == cm0[150:]).all() and (cm[:150] > cm0[:150]).all()


def test_colmass_closed_forms():
    k = np.ones((50, 8))
    q = np.random.default_rng(0).standard_normal((3, 8))
    cm = select.colmass_update(np.zeros(64), q, k, 40)   # identical keys: uniform
    np.testing.assert_allclose(cm[:40], 3 / 40, atol=1e-15)
    k2 = np.zeros((50, 8))
    k2[17, 0] = 1000.0                                   # one overwhelming key
    q2 = np.zeros((1, 8)); q2[0, 0] = 1.0
    cm2 = select.colmass_update(np.zeros(64), q2, k2, 50)
    np.testing.assert_allclose(cm2[17], 1.0, atol=1e-12)
    assert np.argmax(cm2) == 17


def test_select_vertical_multi_head_groups():
    rng = np.random.default_rng(6)
    b, hq, hkv, r, t, d = 2, 4, 2, 3, 96, 32
    q = rng.standard_normal((b, hq, r, d))
    k = rng.standard_normal((b, hkv, t, d))
    cm = np.zeros((b, hkv, t))
    ctx = np.array([96, 70])
    new, sel = select.select_vertical(cm, q, k, ctx, window=16, rho_num=1, rho_den=10)
    # Each KV head received (recent queries x group size) units of mass.
    np.testing.assert_allclose(new.sum(axis=2), r * (hq // hkv), atol=1e-12)
    assert sel[(0, 0)].shape[0] == 8 and sel[(1, 1)].shape[0] == 6
    assert (sel[(1, 1)] < 70 - 16).all()
