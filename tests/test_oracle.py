"""Pins of the fp64 CPU oracle against things other than itself.

* exact integer brute force on the tiny reproduction of PyTorch issue
  #152668 ("Easy repro scenario") and on hundreds of random tiny problems;
* an independent round-to-nearest-even to bf16 (search over the ordered bit
  patterns, exact rational comparisons), and torch's fp32 -> bf16 cast;
* values worked by hand (tests/golden/hand_worked.json);
* closed forms: one-hot rows select a weight row, identity weights copy
  the input, one-row experts give an outer product;
* the three-pass adjoint identity <fwd(X,W), dY> = <X, dgrad(dY,W)> =
  <W, wgrad(X,dY)>, which ties dgrad and wgrad to the forward;
* special cases equal to a library routine: numpy float64 matmul per expert,
  E = 1 is a dense GEMM, equal-size experts are a batched matmul, a fully
  active masked layout is a batched matmul;
* the masked layout compacted into end offsets equals the ragged forward;
* the masked backward (dgrad, wgrad): exact brute force over active rows,
  equality with the ragged passes on the compacted rows, and the adjoint
  identity on the masked layout;
* the SiLU-mul activation on the gate/up forward: torch's SiLU on the exact
  products, the odd and even parts (silu(z) - silu(-z) = z, silu(z) +
  silu(-z) = z tanh(z/2)) via negated gate weights, the gate/up column
  order, and masked = ragged on compacted rows;
* alpha / beta: exact rational brute force of alpha * P + beta * C on every
  pass, beta = 0 never reading C, alpha = 0 returning C, and accumulation
  leaving an empty expert's dW unchanged.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from moe_grouped_gemm_ragged_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers independent of the oracle
# ---------------------------------------------------------------------------

def f32_to_bf16_trunc_bits(values) -> np.ndarray:
    """bf16 bit patterns of values that are exactly bf16 (asserted)."""
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "test value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def bits_to_exact_int(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> Python ints equal to value * 2^133 (every finite bf16 is
    an integer multiple of 2^-133).  Object array, exact."""
    out = np.empty(bits.shape, dtype=object)
    flat_in = bits.ravel()
    flat_out = out.ravel()
    for i, b in enumerate(flat_in):
        b = int(b)
        sign = -1 if b & 0x8000 else 1
        exp = (b >> 7) & 0xFF
        man = b & 0x7F
        assert exp != 0xFF, "finite inputs only"
        if exp == 0:
            val = man                       # man * 2^-133
        else:
            val = (man | 0x80) << (exp - 1)  # (1.man) * 2^(exp-127) * 2^133
        flat_out[i] = sign * val
    return out


SCALE2 = 2 ** 266   # product of two values scaled by 2^133 each


def _bf16_value(bits: int) -> Fraction:
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0:
        return sign * Fraction(man, 2 ** 133)
    return sign * Fraction(man | 0x80, 2 ** 7) * Fraction(2) ** (exp - 127)


_MAX_FINITE = _bf16_value(0x7F7F)
_OVERFLOW_EDGE = _MAX_FINITE + Fraction(2) ** (127 - 8)   # max + half ulp


def rne_bf16_reference(q: Fraction) -> int:
    """Round an exact rational to bf16, nearest with ties to even, by binary
    search over the positive bit patterns (ordered like their values)."""
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    if a >= _OVERFLOW_EDGE:
        return sign | 0x7F80
    lo, hi = 0, 0x7F7F              # invariant: value(lo) <= a
    if a >= _MAX_FINITE:
        return sign | 0x7F7F
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if _bf16_value(mid) <= a:
            lo = mid
        else:
            hi = mid
    if _bf16_value(hi) <= a:
        lo = hi
    if _bf16_value(lo) == a:
        return sign | lo
    up = lo + 1
    dl = a - _bf16_value(lo)
    du = _bf16_value(up) - a
    if dl < du:
        pick = lo
    elif du < dl:
        pick = up
    else:
        pick = lo if lo % 2 == 0 else up
    return sign | pick


def groups_from_offs(offs, m):
    ends, prev = [], 0
    for o in offs:
        e = min(max(int(o), prev), m)
        ends.append(e)
        prev = e
    starts = [0] + ends[:-1]
    return list(zip(starts, ends))


def randn_bf16_bits(rng, shape, std=1.0):
    v = (rng.standard_normal(shape) * std).astype(np.float32)
    u = v.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16   # fp32 -> bf16 RNE for finite values
    return r.astype(np.uint16)


def dec(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# rounding
# ---------------------------------------------------------------------------

def test_round_bf16_matches_exact_reference(oracle_lib):
    rng = np.random.default_rng(123)
    vals = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 130, 3000)))
    # exact ties and near-ties around bf16 values, subnormals and overflow
    for b in [0x0001, 0x0002, 0x007F, 0x0080, 0x3F80, 0x3F81, 0x4049, 0x7F7E, 0x7F7F]:
        v = _bf16_value(b)
        step = _bf16_value(b + 1) - v
        for f in (Fraction(1, 2), Fraction(1, 2) + Fraction(1, 2 ** 40),
                  Fraction(1, 2) - Fraction(1, 2 ** 40), Fraction(1, 3)):
            vals.append(float(v + f * step))
            vals.append(-float(v + f * step))
    vals += [0.0, -0.0, 2.0 ** -134, 2.0 ** -133 * 1.5, 2.0 ** -133 * 2.5,
             3.3895313892515355e38, 3.39e38, 1e300, -1e300]
    got = oracle.round_bf16(np.array(vals))
    for v, g in zip(vals, got):
        want = rne_bf16_reference(Fraction(v))
        if v == 0.0 and np.signbit(v):
            want = 0x8000
        assert int(g) == want, (v, hex(int(g)), hex(want))
    assert oracle.round_bf16(np.array([np.nan]))[0] == 0x7FC0
    assert oracle.round_bf16(np.array([np.inf]))[0] == 0x7F80


def test_round_bf16_matches_torch_on_fp32_values(oracle_lib):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    f = (rng.standard_normal(200000) * np.exp2(rng.integers(-60, 60, 200000))).astype(np.float32)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(f.astype(np.float64))
    np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------------------
# exact brute force
# ---------------------------------------------------------------------------

def exact_ragged(x_bits, w_bits, dy_bits, offs):
    """Exact rational results (as integer numerators over 2^266)."""
    m, k = x_bits.shape
    E, _, n = w_bits.shape
    X = bits_to_exact_int(x_bits)
    W = bits_to_exact_int(w_bits)
    DY = bits_to_exact_int(dy_bits)
    y = {}
    dx = {}
    dw = np.empty((E, k, n), dtype=object)
    for g, (s, e) in enumerate(groups_from_offs(offs, m)):
        for i in range(s, e):
            y[i] = X[i:i + 1].dot(W[g])[0]
            dx[i] = DY[i:i + 1].dot(W[g].T)[0]
        if e > s:
            dw[g] = X[s:e].T.dot(DY[s:e])
        else:
            dw[g] = np.zeros((k, n), dtype=object)
    return y, dx, dw


def _check_exact(value, sabs, exact_num, length):
    """fp64 oracle value vs exact rational; then bf16 rounding vs the
    independent reference."""
    for j in range(len(exact_num)):
        q = Fraction(int(exact_num[j]), SCALE2)
        v = value[j]
        # fp64 summation of exact products: error <= length * 2^-53 * S
        assert abs(Fraction(v) - q) <= Fraction(length) * Fraction(1, 2 ** 52) * Fraction(sabs[j]) , (v, float(q))
        assert oracle.round_bf16_scalar(v) == rne_bf16_reference(q) or q == 0


def test_tiny_repro_config_exact(oracle_lib):
    with open(os.path.join(GOLDEN, "p1_repro.json")) as f:
        g = json.load(f)
    wl = synth.tiny()
    assert list(wl.offs) == g["m_offsets_hang"]
    assert (wl.m, wl.k, wl.n, wl.num_groups) == (g["M"], g["K"], g["N"], g["num_experts"])
    t = synth.make_inputs(wl, "cpu")
    x, w, dy = (synth.bf16_bits(t[a]) for a in ("x", "w", "dy"))
    y_ex, dx_ex, dw_ex = exact_ragged(x, w, dy, wl.offs)
    fw = oracle.forward(x, w, wl.offs)
    dg = oracle.dgrad(dy, w, wl.offs)
    wg = oracle.wgrad(x, dy, wl.offs)
    lo, hi = g["unused_rows"]
    for i in range(wl.m):
        if lo <= i < hi:
            assert fw.status[i] == 0 and dg.status[i] == 0
            assert np.all(np.isnan(fw.value[i]))   # untouched
            continue
        assert fw.status[i] == 1 and dg.status[i] == 1
        _check_exact(fw.value[i], fw.sabs[i], y_ex[i], wl.k)
        _check_exact(dg.value[i], dg.sabs[i], dx_ex[i], wl.n)
    dwv = wg.value.reshape(wl.num_groups, wl.k, wl.n)
    dws = wg.sabs.reshape(wl.num_groups, wl.k, wl.n)
    for gi in range(wl.num_groups):
        for kk in range(wl.k):
            _check_exact(dwv[gi, kk], dws[gi, kk], dw_ex[gi, kk], 32)
    # the empty expert (index 1) has dW == +0.0 exactly, sign bit clear
    assert np.all(dwv[1] == 0.0) and not np.any(np.signbit(dwv[1]))


@pytest.mark.parametrize("seed", range(240))
def test_random_tiny_exact(oracle_lib, seed):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.integers(1, 7))
    k = int(rng.choice([8, 16, 24]))
    n = int(rng.choice([8, 16, 24]))
    sizes = rng.integers(0, 12, E)
    sizes[rng.random(E) < 0.3] = 0            # plenty of empty experts
    if seed % 17 == 0:
        sizes[:] = 0                          # all experts empty
    used = int(sizes.sum())
    m = used + int(rng.integers(0, 6))        # unused trailing rows
    m = max(m, 1)
    offs = np.cumsum(sizes).astype(np.int32)
    x = randn_bf16_bits(rng, (m, k))
    w = randn_bf16_bits(rng, (E, k, n), std=0.5)
    dy = randn_bf16_bits(rng, (m, n))
    y_ex, dx_ex, dw_ex = exact_ragged(x, w, dy, offs)
    fw = oracle.forward(x, w, offs)
    dg = oracle.dgrad(dy, w, offs)
    wg = oracle.wgrad(x, dy, offs)
    for i in range(m):
        if i >= used:
            assert fw.status[i] == 0 and dg.status[i] == 0
            continue
        _check_exact(fw.value[i], fw.sabs[i], y_ex[i], k)
        _check_exact(dg.value[i], dg.sabs[i], dx_ex[i], n)
    dwv = wg.value.reshape(E, k, n)
    dws = wg.sabs.reshape(E, k, n)
    for g in range(E):
        if sizes[g] == 0:
            assert np.all(dwv[g] == 0.0) and not np.any(np.signbit(dwv[g]))
        for kk in range(k):
            _check_exact(dwv[g, kk], dws[g, kk], dw_ex[g, kk], max(int(sizes[g]), 1))
    # masked layout on the same numbers: experts of max_m rows, the first
    # sizes[g] active, inactive rows NaN
    max_m = int(max(int(sizes.max()), 1) + rng.integers(0, 3))
    xm = np.full((E, max_m, k), 0x7FC0, dtype=np.uint16)
    starts = np.concatenate([[0], offs[:-1]])
    for g in range(E):
        xm[g, :sizes[g]] = x[starts[g]:offs[g]]
    mk = oracle.masked_forward(xm, w, sizes.astype(np.int32))
    for g in range(E):
        for r in range(max_m):
            flat = g * max_m + r
            if r < sizes[g]:
                assert mk.status[flat] == 1
                _check_exact(mk.value[flat], mk.sabs[flat], y_ex[starts[g] + r], k)
            else:
                assert mk.status[flat] == 0 and np.all(np.isnan(mk.value[flat]))


# ---------------------------------------------------------------------------
# hand-worked values
# ---------------------------------------------------------------------------

def test_hand_worked_golden(oracle_lib):
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        g = json.load(f)
    r = g["ragged"]
    x = f32_to_bf16_trunc_bits(r["x"])
    w = f32_to_bf16_trunc_bits(r["w"])
    dy = f32_to_bf16_trunc_bits(r["dy"])
    offs = np.array(r["offs"], dtype=np.int32)
    fw = oracle.forward(x, w, offs)
    dg = oracle.dgrad(dy, w, offs)
    wg = oracle.wgrad(x, dy, offs)
    np.testing.assert_array_equal(fw.value[:3], np.array(r["y_rows_0_to_2"], dtype=np.float64))
    np.testing.assert_array_equal(dg.value[:3], np.array(r["dx_rows_0_to_2"], dtype=np.float64))
    np.testing.assert_array_equal(wg.value.reshape(r["E"], r["K"], r["N"]),
                                  np.array(r["dw"], dtype=np.float64))
    for i in r["unused_rows"]:
        assert fw.status[i] == 0 and dg.status[i] == 0
    for e in r["empty_groups"]:
        assert not np.any(np.signbit(wg.value.reshape(r["E"], r["K"], r["N"])[e]))
    mk = g["masked"]
    xm = np.array([[[np.nan if v == "nan" else v for v in row] for row in ex] for ex in mk["x"]],
                  dtype=np.float32)
    xm_bits = xm.view(np.uint32) >> 16
    xm_bits = xm_bits.astype(np.uint16)
    wm = f32_to_bf16_trunc_bits(mk["w"])
    res = oracle.masked_forward(xm_bits, wm, np.array(mk["masked_m"], dtype=np.int32))
    for key, want in mk["y_active"].items():
        e, row = map(int, key.split(","))
        np.testing.assert_array_equal(res.value[e * mk["max_m"] + row], np.array(want, dtype=np.float64))
    for key in mk["inactive"]:
        e, row = map(int, key.split(","))
        assert res.status[e * mk["max_m"] + row] == 0


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def test_one_hot_rows_select_weight_rows(oracle_lib):
    rng = np.random.default_rng(5)
    E, k, n = 3, 16, 24
    sizes = [5, 0, 11]
    offs = np.cumsum(sizes).astype(np.int32)
    m = int(offs[-1])
    w = randn_bf16_bits(rng, (E, k, n))
    x = np.zeros((m, k), dtype=np.uint16)
    pick = rng.integers(0, k, m)
    x[np.arange(m), pick] = 0x3F80            # 1.0
    fw = oracle.forward(x, w, offs)
    for g, (s, e) in enumerate(groups_from_offs(offs, m)):
        for i in range(s, e):
            np.testing.assert_array_equal(fw.value[i], dec(w[g, pick[i]]))


def test_identity_weights_copy_input(oracle_lib):
    rng = np.random.default_rng(6)
    E, k = 4, 16
    sizes = [3, 7, 0, 6]
    offs = np.cumsum(sizes).astype(np.int32)
    m = int(offs[-1]) + 2
    x = randn_bf16_bits(rng, (m, k))
    w = np.zeros((E, k, k), dtype=np.uint16)
    for g in range(E):
        w[g][np.arange(k), np.arange(k)] = 0x3F80
    fw = oracle.forward(x, w, offs)
    dg = oracle.dgrad(x, w, offs)               # W^T = I as well
    for i in range(int(offs[-1])):
        np.testing.assert_array_equal(fw.value[i], dec(x[i]))
        np.testing.assert_array_equal(dg.value[i], dec(x[i]))
    assert fw.status[-1] == 0 and fw.status[-2] == 0


def test_one_row_experts_give_outer_products(oracle_lib):
    rng = np.random.default_rng(8)
    E, k, n = 5, 8, 16
    offs = np.array([1, 2, 2, 3, 4], dtype=np.int32)   # expert 2 empty
    x = randn_bf16_bits(rng, (4, k))
    dy = randn_bf16_bits(rng, (4, n))
    wg = oracle.wgrad(x, dy, offs).value.reshape(E, k, n)
    rows = {0: 0, 1: 1, 3: 2, 4: 3}
    for g in range(E):
        if g in rows:
            i = rows[g]
            np.testing.assert_array_equal(wg[g], np.outer(dec(x[i]), dec(dy[i])))
        else:
            assert np.all(wg[g] == 0.0) and not np.any(np.signbit(wg[g]))


def test_invalid_offsets_are_clamped(oracle_lib):
    """Decreasing offsets give empty experts; offsets past M are cut at M."""
    rng = np.random.default_rng(9)
    m, k, n = 10, 8, 8
    offs = np.array([4, 2, 7, 30], dtype=np.int32)   # -> groups [0,4) [4,4) [4,7) [7,10)
    x = randn_bf16_bits(rng, (m, k))
    w = randn_bf16_bits(rng, (4, k, n))
    dy = randn_bf16_bits(rng, (m, n))
    fw = oracle.forward(x, w, offs)
    want_g = [0] * 4 + [2] * 3 + [3] * 3
    for i in range(m):
        assert fw.status[i] == 1
        np.testing.assert_allclose(fw.value[i], dec(x[i]) @ dec(w[want_g[i]]), rtol=1e-13, atol=1e-13)
    wg = oracle.wgrad(x, dy, offs).value.reshape(4, k, n)
    assert np.all(wg[1] == 0.0)


# ---------------------------------------------------------------------------
# library special cases and identities on medium problems
# ---------------------------------------------------------------------------

def _medium(name):
    wl = synth.by_name(name)
    t = synth.make_inputs(wl, "cpu", need=("x", "w") if wl.layout == "masked" else ("x", "w", "dy"))
    return wl, {kk: (synth.bf16_bits(v) if kk in ("x", "w", "dy") else v.numpy()) for kk, v in t.items()}


@pytest.mark.parametrize("name", ["qwen3_gateup_small", "dsv3_small", "glm_up_small"])
def test_matches_numpy_per_expert_matmul(oracle_lib, name):
    wl, t = _medium(name)
    x, w, dy, offs = t["x"], t["w"], t["dy"], t["offs"]
    X, Wd, DY = dec(x), dec(w), dec(dy)
    fw = oracle.forward(x, w, offs)
    dg = oracle.dgrad(dy, w, offs)
    wg = oracle.wgrad(x, dy, offs)
    dwv = wg.value.reshape(wl.num_groups, wl.k, wl.n)
    dws = wg.sabs.reshape(wl.num_groups, wl.k, wl.n)
    for g, (s, e) in enumerate(groups_from_offs(offs, wl.m)):
        ref_y = X[s:e] @ Wd[g]
        ref_dx = DY[s:e] @ Wd[g].T
        ref_dw = X[s:e].T @ DY[s:e]
        tol = 1e-13
        assert np.all(np.abs(fw.value[s:e] - ref_y) <= tol * fw.sabs[s:e] + 1e-300)
        assert np.all(np.abs(dg.value[s:e] - ref_dx) <= tol * dg.sabs[s:e] + 1e-300)
        assert np.all(np.abs(dwv[g] - ref_dw) <= tol * dws[g] + 1e-300)
        # |X||W| is S computed by a library routine
        np.testing.assert_allclose(fw.sabs[s:e], np.abs(X[s:e]) @ np.abs(Wd[g]), rtol=1e-12)


def test_single_expert_is_dense_gemm(oracle_lib):
    rng = np.random.default_rng(11)
    m, k, n = 37, 40, 24
    x = randn_bf16_bits(rng, (m, k))
    w = randn_bf16_bits(rng, (1, k, n))
    dy = randn_bf16_bits(rng, (m, n))
    offs = np.array([m], dtype=np.int32)
    np.testing.assert_allclose(oracle.forward(x, w, offs).value, dec(x) @ dec(w[0]), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.dgrad(dy, w, offs).value, dec(dy) @ dec(w[0]).T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.wgrad(x, dy, offs).value, dec(x).T @ dec(dy), rtol=1e-12, atol=1e-12)


def test_equal_experts_are_batched_matmul(oracle_lib):
    rng = np.random.default_rng(12)
    E, r, k, n = 6, 9, 16, 32
    x = randn_bf16_bits(rng, (E * r, k))
    w = randn_bf16_bits(rng, (E, k, n))
    dy = randn_bf16_bits(rng, (E * r, n))
    offs = (np.arange(1, E + 1) * r).astype(np.int32)
    Xb = dec(x).reshape(E, r, k)
    DYb = dec(dy).reshape(E, r, n)
    np.testing.assert_allclose(oracle.forward(x, w, offs).value.reshape(E, r, n),
                               np.matmul(Xb, dec(w)), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.wgrad(x, dy, offs).value.reshape(E, k, n),
                               np.matmul(Xb.transpose(0, 2, 1), DYb), rtol=1e-12, atol=1e-12)
    # masked layout with every row active is the same batched matmul
    res = oracle.masked_forward(x.reshape(E, r, k), w, np.full(E, r, dtype=np.int32))
    np.testing.assert_allclose(res.value.reshape(E, r, n), np.matmul(Xb, dec(w)), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("name", ["qwen3_gateup_small", "dsv3_small", "tiny"])
def test_adjoint_identity(oracle_lib, name):
    """<fwd(X,W), dY> = <X, dgrad(dY,W)> = <W, wgrad(X,dY)> over the rows
    that belong to experts (all three are sum_g sum_{i in g} X W dY)."""
    wl, t = _medium(name) if name != "tiny" else (synth.tiny(), None)
    if t is None:
        tt = synth.make_inputs(wl, "cpu")
        t = {kk: (synth.bf16_bits(v) if kk in ("x", "w", "dy") else v.numpy()) for kk, v in tt.items()}
    x, w, dy, offs = t["x"], t["w"], t["dy"], t["offs"]
    fw = oracle.forward(x, w, offs)
    dg = oracle.dgrad(dy, w, offs)
    wg = oracle.wgrad(x, dy, offs)
    used = fw.status == 1
    a = np.sum(fw.value[used] * dec(dy)[used])
    b = np.sum(dec(x)[used] * dg.value[used])
    c = np.sum(dec(w) * wg.value.reshape(wl.num_groups, wl.k, wl.n))
    scale = np.sum(np.abs(fw.value[used]) * np.abs(dec(dy)[used])) + 1e-300
    assert abs(a - b) <= 1e-10 * scale
    assert abs(a - c) <= 1e-10 * scale


def test_masked_compacts_to_ragged(oracle_lib):
    """Masked rows r < masked_m[e] equal the ragged forward of the same rows
    stacked with end offsets cumsum(masked_m) -- bit-exactly."""
    wl, t = _medium("masked_down_small")
    x, w, mm = t["x"], t["w"], t["masked_m"]
    sizes = wl.group_sizes()
    res = oracle.masked_forward(x, w, mm)
    xr = np.concatenate([x[e, :sizes[e]] for e in range(wl.num_groups)], axis=0)
    offs = np.cumsum(sizes).astype(np.int32)
    fw = oracle.forward(xr, w, offs)
    row = 0
    for e in range(wl.num_groups):
        for r in range(wl.m):
            flat = e * wl.m + r
            if r < sizes[e]:
                assert res.status[flat] == 1
                np.testing.assert_array_equal(res.value[flat], fw.value[row])
                row += 1
            else:
                assert res.status[flat] == 0
    # inactive rows of X are NaN in this workload and nothing leaked
    assert np.all(np.isfinite(res.value[res.status == 1]))


def test_masked_count_clamped(oracle_lib):
    rng = np.random.default_rng(13)
    E, max_m, k, n = 3, 4, 8, 8
    x = randn_bf16_bits(rng, (E, max_m, k))
    w = randn_bf16_bits(rng, (E, k, n))
    res = oracle.masked_forward(x, w, np.array([-3, 99, 2], dtype=np.int32))
    st = res.status.reshape(E, max_m)
    assert st[0].sum() == 0 and st[1].sum() == max_m and list(st[2]) == [1, 1, 0, 0]


def test_sampled_rows_equal_full(oracle_lib):
    wl, t = _medium("dsv3_small")
    x, w, dy, offs = t["x"], t["w"], t["dy"], t["offs"]
    full = oracle.forward(x, w, offs)
    rows = np.array([0, 5, wl.m - 1, 77, 1000])
    part = oracle.forward(x, w, offs, rows=rows)
    np.testing.assert_array_equal(part.value, full.value[rows])
    wfull = oracle.wgrad(x, dy, offs)
    pairs = np.array([[0, 0], [3, 17], [wl.num_groups - 1, wl.k - 1]])
    wpart = oracle.wgrad(x, dy, offs, pairs=pairs)
    for j, (g, kk) in enumerate(pairs):
        np.testing.assert_array_equal(wpart.value[j], wfull.value[g * wl.k + kk])


# ---------------------------------------------------------------------------
# alpha / beta: out = alpha * P + beta * C with one rounding (fused
# accumulation; TransformerEngine PR #3542, "Changes")
# ---------------------------------------------------------------------------

ALPHA_BETA = [(1.0, 1.0), (-0.5, 2.0), (0.25, -1.0), (3.0, 0.5), (0.0, 1.0), (2.0, 0.0)]


def _check_exact_ab(value, sabs, exact_num, c_vals, alpha, beta, length):
    """fp64 oracle value vs the exact rational alpha * P + beta * C, then its
    bf16 rounding vs the independent reference."""
    for j in range(len(exact_num)):
        q = Fraction(alpha) * Fraction(int(exact_num[j]), SCALE2)
        if beta != 0.0:
            q += Fraction(beta) * Fraction(float(c_vals[j]))
        v = value[j]
        assert abs(Fraction(v) - q) <= Fraction(length + 1) * Fraction(1, 2 ** 52) * Fraction(sabs[j]), (v, float(q))
        assert oracle.round_bf16_scalar(v) == rne_bf16_reference(q) or q == 0


@pytest.mark.parametrize("alpha,beta", ALPHA_BETA)
@pytest.mark.parametrize("seed", range(6))
def test_alpha_beta_exact(oracle_lib, seed, alpha, beta):
    rng = np.random.default_rng(5000 + seed)
    E = int(rng.integers(1, 5))
    k = int(rng.choice([8, 16]))
    n = int(rng.choice([8, 16]))
    sizes = rng.integers(0, 9, E)
    sizes[rng.random(E) < 0.3] = 0
    used = int(sizes.sum())
    m = max(used + int(rng.integers(0, 4)), 1)
    offs = np.cumsum(sizes).astype(np.int32)
    x = randn_bf16_bits(rng, (m, k))
    w = randn_bf16_bits(rng, (E, k, n), std=0.5)
    dy = randn_bf16_bits(rng, (m, n))
    cy = randn_bf16_bits(rng, (m, n), std=4.0)          # prior Y (bf16 output)
    cx = randn_bf16_bits(rng, (m, k), std=4.0)          # prior dX
    cw = (rng.standard_normal((E * k, n)) * 3).astype(np.float32)   # prior dW (fp32 output)
    y_ex, dx_ex, dw_ex = exact_ragged(x, w, dy, offs)
    fw = oracle.forward(x, w, offs, alpha=alpha, beta=beta, c_in=cy)
    dg = oracle.dgrad(dy, w, offs, alpha=alpha, beta=beta, c_in=cx)
    wg = oracle.wgrad(x, dy, offs, alpha=alpha, beta=beta, c_in=cw)
    for i in range(used):
        _check_exact_ab(fw.value[i], fw.sabs[i], y_ex[i], dec(cy[i]), alpha, beta, k)
        _check_exact_ab(dg.value[i], dg.sabs[i], dx_ex[i], dec(cx[i]), alpha, beta, n)
    for i in range(used, m):
        assert fw.status[i] == 0 and np.all(np.isnan(fw.value[i]))
    dwv = wg.value.reshape(E, k, n)
    dws = wg.sabs.reshape(E, k, n)
    cwv = cw.reshape(E, k, n)
    for g in range(E):
        for kk in range(k):
            _check_exact_ab(dwv[g, kk], dws[g, kk], dw_ex[g, kk], cwv[g, kk], alpha, beta,
                            max(int(sizes[g]), 1))
    # masked layout on the same numbers
    max_m = int(max(int(sizes.max()), 1))
    xm = np.full((E, max_m, k), 0x7FC0, dtype=np.uint16)
    cm = np.full((E * max_m, n), 0x7FC0, dtype=np.uint16)
    starts = np.concatenate([[0], offs[:-1]])
    for g in range(E):
        xm[g, :sizes[g]] = x[starts[g]:offs[g]]
        cm[g * max_m:g * max_m + sizes[g]] = cy[starts[g]:offs[g]]
    mk = oracle.masked_forward(xm, w, sizes.astype(np.int32), alpha=alpha, beta=beta, c_in=cm)
    for g in range(E):
        for r in range(int(sizes[g])):
            flat = g * max_m + r
            _check_exact_ab(mk.value[flat], mk.sabs[flat], y_ex[starts[g] + r], dec(cy[starts[g] + r]),
                            alpha, beta, k)


def test_beta_zero_never_reads_prior_output(oracle_lib):
    rng = np.random.default_rng(77)
    x = randn_bf16_bits(rng, (20, 16))
    w = randn_bf16_bits(rng, (3, 16, 8))
    offs = np.array([5, 5, 18], dtype=np.int32)
    nan_c = np.full((20, 8), 0x7FC0, dtype=np.uint16)
    a = oracle.forward(x, w, offs, alpha=-2.0, beta=0.0, c_in=nan_c)
    b = oracle.forward(x, w, offs)
    ok = b.status == 1
    assert np.array_equal(a.value[ok], -2.0 * b.value[ok])
    assert np.all(np.isfinite(a.value[ok]))


def test_alpha_zero_beta_one_returns_prior_output(oracle_lib):
    rng = np.random.default_rng(78)
    x = randn_bf16_bits(rng, (20, 16))
    dy = randn_bf16_bits(rng, (20, 8))
    offs = np.array([5, 5, 18], dtype=np.int32)
    c = (rng.standard_normal((3 * 16, 8)) * 5).astype(np.float32)
    r = oracle.wgrad(x, dy, offs, alpha=0.0, beta=1.0, c_in=c)
    assert np.array_equal(r.value, c.astype(np.float64))


def test_accumulating_wgrad_keeps_empty_experts(oracle_lib):
    """dW[g] += X_g^T dY_g: an expert with no rows keeps its prior dW."""
    rng = np.random.default_rng(79)
    x = randn_bf16_bits(rng, (12, 8))
    dy = randn_bf16_bits(rng, (12, 8))
    offs = np.array([0, 7, 7, 12], dtype=np.int32)
    c = (rng.standard_normal((4 * 8, 8))).astype(np.float32)
    acc = oracle.wgrad(x, dy, offs, alpha=1.0, beta=1.0, c_in=c).value.reshape(4, 8, 8)
    plain = oracle.wgrad(x, dy, offs).value.reshape(4, 8, 8)
    cc = c.astype(np.float64).reshape(4, 8, 8)
    for g in (0, 2):
        assert np.array_equal(acc[g], cc[g])
    for g in (1, 3):
        assert np.allclose(acc[g], plain[g] + cc[g], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# masked dgrad / wgrad: the backward of the masked forward over active rows
# (sglang PR #32385, "Evidence" and "Cause")
# ---------------------------------------------------------------------------

def _masked_case(rng, E, max_m, k, n):
    act = rng.integers(0, max_m + 1, E)
    act[rng.random(E) < 0.25] = 0
    dy = np.full((E, max_m, n), 0x7FC0, dtype=np.uint16)     # NaN in inactive rows
    x = np.full((E, max_m, k), 0x7FC0, dtype=np.uint16)
    for e in range(E):
        dy[e, :act[e]] = randn_bf16_bits(rng, (int(act[e]), n))
        x[e, :act[e]] = randn_bf16_bits(rng, (int(act[e]), k))
    w = randn_bf16_bits(rng, (E, k, n), std=0.5)
    return act.astype(np.int32), x, dy, w


@pytest.mark.parametrize("seed", range(30))
def test_masked_backward_exact(oracle_lib, seed):
    rng = np.random.default_rng(7000 + seed)
    E = int(rng.integers(1, 5))
    max_m = int(rng.integers(1, 9))
    k = int(rng.choice([8, 16]))
    n = int(rng.choice([8, 16]))
    act, x, dy, w = _masked_case(rng, E, max_m, k, n)
    dg = oracle.masked_dgrad(dy, w, act)
    wg = oracle.masked_wgrad(x, dy, act)
    W = bits_to_exact_int(w)
    for e in range(E):
        DY = bits_to_exact_int(dy[e, :act[e]])
        X = bits_to_exact_int(x[e, :act[e]])
        for r in range(max_m):
            flat = e * max_m + r
            if r < act[e]:
                assert dg.status[flat] == 1
                _check_exact(dg.value[flat], dg.sabs[flat], DY[r:r + 1].dot(W[e].T)[0], n)
            else:
                assert dg.status[flat] == 0 and np.all(np.isnan(dg.value[flat]))
        dwe = X.T.dot(DY) if act[e] > 0 else np.zeros((k, n), dtype=object)
        for kk in range(k):
            row = e * k + kk
            _check_exact(wg.value[row], wg.sabs[row], dwe[kk], max(int(act[e]), 1))
        if act[e] == 0:
            v = wg.value[e * k:(e + 1) * k]
            assert np.all(v == 0.0) and not np.any(np.signbit(v))


def test_masked_backward_compacts_to_ragged(oracle_lib):
    """The masked passes on active rows equal the ragged passes on the same
    rows packed densely (offsets = cumsum(masked_m))."""
    rng = np.random.default_rng(91)
    E, max_m, k, n = 5, 24, 32, 40
    act, x, dy, w = _masked_case(rng, E, max_m, k, n)
    xr = np.concatenate([x[e, :act[e]] for e in range(E)])
    dyr = np.concatenate([dy[e, :act[e]] for e in range(E)])
    offs = np.cumsum(act).astype(np.int32)
    mdg = oracle.masked_dgrad(dy, w, act)
    rdg = oracle.dgrad(dyr, w, offs)
    mwg = oracle.masked_wgrad(x, dy, act)
    rwg = oracle.wgrad(xr, dyr, offs)
    flat = np.concatenate([np.arange(act[e]) + e * max_m for e in range(E)])
    assert np.array_equal(mdg.value[flat], rdg.value)
    assert np.array_equal(mwg.value, rwg.value)


def test_masked_adjoint_identity(oracle_lib):
    """<fwd(X,W), dY> = <X, dgrad(dY,W)> = <W, wgrad(X,dY)> on active rows."""
    rng = np.random.default_rng(92)
    E, max_m, k, n = 4, 16, 24, 32
    act, x, dy, w = _masked_case(rng, E, max_m, k, n)
    fw = oracle.masked_forward(x, w, act)
    dg = oracle.masked_dgrad(dy, w, act)
    wg = oracle.masked_wgrad(x, dy, act)
    ok = fw.status == 1
    X, DY, W = dec(x).reshape(E * max_m, k), dec(dy).reshape(E * max_m, n), dec(w).reshape(E * k, n)
    a = float(np.sum(fw.value[ok] * DY[ok]))
    b = float(np.sum(X[ok] * dg.value[ok]))
    c = float(np.sum(W * wg.value))
    assert abs(a - b) <= 1e-9 * max(1.0, abs(a)) and abs(a - c) <= 1e-9 * max(1.0, abs(a))


# ---------------------------------------------------------------------------
# SiLU-mul activation on the gate/up forward (sglang PR #32385, "Cause")
# ---------------------------------------------------------------------------

def _silu_case(seed, E=3, k=16, i=8):
    rng = np.random.default_rng(seed)
    sizes = np.array([5, 0, 9][:E])
    offs = np.cumsum(sizes).astype(np.int32)
    m = int(offs[-1]) + 2
    x = randn_bf16_bits(rng, (m, k))
    w13 = randn_bf16_bits(rng, (E, k, 2 * i))
    return x, w13, offs, i


def test_silu_mul_matches_library_silu(oracle_lib):
    """torch's SiLU in fp64 on the oracle's exact gate and up products."""
    torch = pytest.importorskip("torch")
    x, w13, offs, i = _silu_case(1)
    r = oracle.forward_silu_mul(x, w13, offs)
    g = oracle.forward(x, np.ascontiguousarray(w13[:, :, :i]), offs)
    u = oracle.forward(x, np.ascontiguousarray(w13[:, :, i:]), offs)
    ok = r.status == 1
    lib = torch.nn.functional.silu(torch.from_numpy(g.value[ok])).numpy() * u.value[ok]
    assert np.allclose(r.value[ok], lib, rtol=1e-13, atol=0)
    assert np.all(r.status == g.status)


def test_silu_odd_part_is_identity(oracle_lib):
    """silu(z) - silu(-z) = z: negating the gate weights negates the gate
    exactly, so out(W) - out(W with -gate) = gate * up."""
    x, w13, offs, i = _silu_case(2)
    neg = w13.copy()
    neg[:, :, :i] ^= 0x8000
    a = oracle.forward_silu_mul(x, w13, offs)
    b = oracle.forward_silu_mul(x, neg, offs)
    g = oracle.forward(x, np.ascontiguousarray(w13[:, :, :i]), offs)
    u = oracle.forward(x, np.ascontiguousarray(w13[:, :, i:]), offs)
    ok = a.status == 1
    want = g.value[ok] * u.value[ok]
    assert np.allclose(a.value[ok] - b.value[ok], want, rtol=1e-12, atol=1e-12)


def test_silu_even_part_is_tanh(oracle_lib):
    """silu(z) + silu(-z) = z tanh(z / 2)."""
    x, w13, offs, i = _silu_case(3)
    neg = w13.copy()
    neg[:, :, :i] ^= 0x8000
    a = oracle.forward_silu_mul(x, w13, offs)
    b = oracle.forward_silu_mul(x, neg, offs)
    g = oracle.forward(x, np.ascontiguousarray(w13[:, :, :i]), offs)
    u = oracle.forward(x, np.ascontiguousarray(w13[:, :, i:]), offs)
    ok = a.status == 1
    want = g.value[ok] * np.tanh(g.value[ok] / 2) * u.value[ok]
    assert np.allclose(a.value[ok] + b.value[ok], want, rtol=1e-12, atol=1e-12)


def test_silu_zero_gate_gives_zero_and_layout(oracle_lib):
    """Gate weights of zero give silu(0) = 0 whatever the up half holds; and
    the gate is the FIRST half of the columns: zeroing the second half
    (the up projection) zeroes the output instead."""
    x, w13, offs, i = _silu_case(4)
    zg = w13.copy()
    zg[:, :, :i] = 0
    r = oracle.forward_silu_mul(x, zg, offs)
    ok = r.status == 1
    assert np.all(r.value[ok] == 0.0)
    zu = w13.copy()
    zu[:, :, i:] = 0
    r2 = oracle.forward_silu_mul(x, zu, offs)
    assert np.all(r2.value[ok] == 0.0)
    assert np.any(oracle.forward_silu_mul(x, w13, offs).value[ok] != 0.0)


def test_masked_silu_mul_compacts_to_ragged(oracle_lib):
    rng = np.random.default_rng(95)
    E, max_m, k, i = 4, 12, 16, 8
    act = np.array([3, 0, 12, 7], dtype=np.int32)
    x = np.full((E, max_m, k), 0x7FC0, dtype=np.uint16)
    for e in range(E):
        x[e, :act[e]] = randn_bf16_bits(rng, (int(act[e]), k))
    w13 = randn_bf16_bits(rng, (E, k, 2 * i))
    m = oracle.masked_forward_silu_mul(x, w13, act)
    xr = np.concatenate([x[e, :act[e]] for e in range(E)])
    r = oracle.forward_silu_mul(xr, w13, np.cumsum(act).astype(np.int32))
    flat = np.concatenate([np.arange(act[e]) + e * max_m for e in range(E)])
    assert np.array_equal(m.value[flat], r.value)
    assert int((m.status == 1).sum()) == int(act.sum())
