"""Pins of the oracle's [E, N, K] weight-layout functions: exact rational
brute force written against the [E, N, K] indexing directly (W[g, n, k]),
independent of the [E, K, N] functions they are built on."""
from fractions import Fraction

import numpy as np

import oracle


def bits(rng, shape):
    """Small dyadic bf16 values (exact): integers -8..8 times 2^-3."""
    v = rng.integers(-8, 9, size=shape).astype(np.float32) / 8.0
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def val(b):
    return Fraction(float(oracle.decode_bf16(np.array([b]))[0]))


OFFS = np.array([3, 3, 7], dtype=np.int32)      # expert 1 empty, rows 7, 8 unused
OWNER = [0, 0, 0, 2, 2, 2, 2, None, None]


def test_forward_nk_brute_force():
    rng = np.random.default_rng(1)
    m, k, n, e = 9, 5, 4, 3
    x, w = bits(rng, (m, k)), bits(rng, (e, n, k))
    res = oracle.forward_nk(x, w, OFFS)
    for i in range(m):
        g = OWNER[i]
        assert res.status[i] == (g is not None)
        if g is None:
            continue
        for j in range(n):
            assert Fraction(res.value[i, j]) == sum(val(x[i, kk]) * val(w[g, j, kk]) for kk in range(k))


def test_dgrad_nk_brute_force():
    rng = np.random.default_rng(2)
    m, k, n, e = 9, 5, 4, 3
    dy, w = bits(rng, (m, n)), bits(rng, (e, n, k))
    res = oracle.dgrad_nk(dy, w, OFFS)
    for i in range(m):
        g = OWNER[i]
        if g is None:
            assert res.status[i] == 0
            continue
        for kk in range(k):
            assert Fraction(res.value[i, kk]) == sum(val(dy[i, j]) * val(w[g, j, kk]) for j in range(n))


def test_wgrad_nk_brute_force():
    rng = np.random.default_rng(3)
    m, k, n, e = 9, 5, 4, 3
    x, dy = bits(rng, (m, k)), bits(rng, (m, n))
    res = oracle.wgrad_nk(x, dy, OFFS)
    for g in range(e):
        rows = [i for i in range(m) if OWNER[i] == g]
        for j in range(n):
            r = g * n + j
            assert tuple(res.index[r]) == (g, j)
            for kk in range(k):
                want = sum((val(dy[i, j]) * val(x[i, kk]) for i in rows), Fraction(0))
                assert Fraction(res.value[r, kk]) == want
                if not rows:
                    assert res.value[r, kk] == 0.0 and not np.signbit(res.value[r, kk])


def test_masked_forward_nk_brute_force():
    rng = np.random.default_rng(4)
    e, max_m, k, n = 3, 4, 5, 3
    mm = np.array([2, 0, 4], dtype=np.int32)
    x, w = bits(rng, (e, max_m, k)), bits(rng, (e, n, k))
    res = oracle.masked_forward_nk(x, w, mm)
    for ex in range(e):
        for r in range(max_m):
            flat = ex * max_m + r
            assert res.status[flat] == (r < mm[ex])
            if r < mm[ex]:
                for j in range(n):
                    assert Fraction(res.value[flat, j]) == sum(
                        val(x[ex, r, kk]) * val(w[ex, j, kk]) for kk in range(k))
