"""Pins of the oracle's grouped bias with a per-token factor: exact rational
brute force of alpha * X W[g] + beta * C + s[i] * bias[g] on the ragged and
masked layouts, with unused capacity rows (status 0, their factors never
read: the factor array holds only the logical rows) and s = None meaning 1;
and its backward (dbias, ds) by the same brute force."""
from fractions import Fraction

import numpy as np

import oracle


def bits(rng, shape):
    v = rng.integers(-8, 9, size=shape).astype(np.float32) / 8.0
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def val(b):
    return Fraction(float(oracle.decode_bf16(np.array([b]))[0]))


def test_forward_bias_brute_force_with_capacity():
    rng = np.random.default_rng(11)
    m, k, n, e = 10, 5, 4, 3
    offs = np.array([3, 3, 7], dtype=np.int32)       # expert 1 empty; rows 7..9 are capacity
    owner = [0, 0, 0, 2, 2, 2, 2]
    x, w = bits(rng, (m, k)), bits(rng, (e, k, n))
    bias = bits(rng, (e, n))
    scale = (rng.integers(-4, 5, size=7) / 4.0).astype(np.float32)   # logical rows only
    c = bits(rng, (m, n))
    res = oracle.forward_bias(x, w, offs, bias, scale, alpha=0.5, beta=-2.0, c_in=c)
    for i in range(m):
        if i >= 7:
            assert res.status[i] == 0
            continue
        g = owner[i]
        for j in range(n):
            want = (Fraction(1, 2) * sum(val(x[i, kk]) * val(w[g, kk, j]) for kk in range(k))
                    - 2 * val(c[i, j]) + Fraction(float(scale[i])) * val(bias[g, j]))
            assert Fraction(res.value[i, j]) == want
    plain = oracle.forward_bias(x, w, offs, bias, None)
    for i in range(7):
        g = owner[i]
        for j in range(n):
            assert Fraction(plain.value[i, j]) == sum(
                val(x[i, kk]) * val(w[g, kk, j]) for kk in range(k)) + val(bias[g, j])


def test_masked_forward_bias_brute_force():
    rng = np.random.default_rng(12)
    e, max_m, k, n = 3, 4, 5, 3
    mm = np.array([2, 0, 4], dtype=np.int32)
    x, w = bits(rng, (e, max_m, k)), bits(rng, (e, k, n))
    bias = bits(rng, (e, n))
    scale = (rng.integers(-4, 5, size=(e, max_m)) / 4.0).astype(np.float32)
    scale[0, 2:] = np.nan                      # inactive factors are never read
    res = oracle.masked_forward_bias(x, w, mm, bias, scale)
    for ex in range(e):
        for r in range(max_m):
            flat = ex * max_m + r
            if r >= mm[ex]:
                assert res.status[flat] == 0
                continue
            for j in range(n):
                want = sum(val(x[ex, r, kk]) * val(w[ex, kk, j]) for kk in range(k)) \
                    + Fraction(float(scale[ex, r])) * val(bias[ex, j])
                assert Fraction(res.value[flat, j]) == want


def test_bias_grad_brute_force():
    rng = np.random.default_rng(13)
    m, n, e = 9, 4, 3
    offs = np.array([3, 3, 7], dtype=np.int32)
    owner = [0, 0, 0, 2, 2, 2, 2, None, None]
    dy = bits(rng, (m, n))
    s = (rng.integers(-4, 5, size=7) / 4.0).astype(np.float32)      # logical rows only
    res = oracle.bias_grad(dy, offs, s)
    for g in range(e):
        rows = [i for i in range(m) if owner[i] == g]
        for j in range(n):
            want = sum((Fraction(float(s[i])) * val(dy[i, j]) for i in rows), Fraction(0))
            assert Fraction(res.value[g, j]) == want
    assert np.all(res.value[1] == 0.0) and not np.any(np.signbit(res.value[1]))
    plain = oracle.bias_grad(dy, offs, None)
    assert Fraction(plain.value[0, 0]) == sum(val(dy[i, 0]) for i in range(3))


def test_bias_scale_grad_brute_force():
    """ds and the masked dbias pinned by brute force; rows no expert owns
    (and inactive masked rows) have status 0."""
    rng = np.random.default_rng(14)
    m, n, e = 9, 4, 3
    offs = np.array([3, 3, 7], dtype=np.int32)
    owner = [0, 0, 0, 2, 2, 2, 2, None, None]
    dy, bias = bits(rng, (m, n)), bits(rng, (e, n))
    res = oracle.bias_scale_grad(dy, offs, bias)
    for i in range(m):
        if owner[i] is None:
            assert res.status[i] == 0
            continue
        assert Fraction(res.value[i, 0]) == sum(val(bias[owner[i], j]) * val(dy[i, j]) for j in range(n))
    # masked layout
    mm = np.array([2, 0, 3], dtype=np.int32)
    dym = bits(rng, (e, 3, n))
    rm = oracle.bias_scale_grad(dym, mm, bias, masked=True)
    assert rm.status.tolist() == [1, 1, 0, 0, 0, 0, 1, 1, 1]
    gm = oracle.bias_grad(dym, mm, None, masked=True)
    assert Fraction(gm.value[2, 1]) == sum(val(dym[2, r, 1]) for r in range(3))
    assert np.all(gm.value[1] == 0.0)
