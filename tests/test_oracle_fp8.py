"""Pins of the fp8 block-scaled oracle against things other than itself.

* the e4m3 decoding of all 256 codes against torch's float8_e4m3fn cast
  (a library routine), and a few codes worked from the format's definition;
* exact rational brute force (fractions, values decoded by torch) on tiny
  ragged and masked problems, within the fp64 summation bound;
* the block index of the scales: a scale of k-block 1 multiplies exactly the
  k in [128, 256) (numpy float64 matmul on the torch-decoded partial sums);
* numpy float64 matmul per expert on torch-decoded, scale-expanded operands;
* the masked layout: inactive rows (NaN codes and non-power-of-two scales)
  are never read, and masked = ragged on the compacted rows;
* the UE8M0 validity count against hand-picked fp32 bit patterns.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_ragged_amd import synth


def torch_e4m3(codes) -> np.ndarray:
    """Library decoding: torch's float8_e4m3fn -> float64."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def rand_codes(rng, shape) -> np.ndarray:
    """Random e4m3 codes without the two NaN codes."""
    c = rng.integers(0, 256, size=shape, dtype=np.int64)
    c = np.where((c & 0x7F) == 0x7F, c - 1, c)
    return c.astype(np.uint8)


def rand_pow2(rng, shape, lo=-8, hi=4) -> np.ndarray:
    return np.ldexp(1.0, rng.integers(lo, hi + 1, size=shape)).astype(np.float32)


def expand(scales, k) -> np.ndarray:
    """[..., G] block scales -> [..., K], each repeated over its 128 values."""
    return np.repeat(np.asarray(scales, dtype=np.float64), 128, axis=-1)[..., :k]


# --------------------------------------------------------------------------
# e4m3 codec
# --------------------------------------------------------------------------

def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch_e4m3(codes)
    got = np.array([oracle.decode_e4m3(c) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x40, 2.0), (0x77, 240.0), (0x7E, 448.0), (0xB8, -1.0),
    (0xFE, -448.0), (0x3C, 1.5)])
def test_e4m3_decode_closed_forms(code, value):
    # normal: (1 + m/8) 2^(e-7); subnormal: m 2^-9 (OCP E4M3)
    assert oracle.decode_e4m3(code) == value


# --------------------------------------------------------------------------
# forward: brute force, block index, library matmul
# --------------------------------------------------------------------------

def exact_row(xc, sxr, wc, swr):
    """Exact value of one output element set: Fractions of torch-decoded
    codes and the scales."""
    xv = torch_e4m3(xc)
    wv = torch_e4m3(wc)
    k = len(xv)
    out = []
    for j in range(wv.shape[0]):
        acc = Fraction(0)
        for kk in range(k):
            acc += (Fraction(float(xv[kk])) * Fraction(float(sxr[kk // 128]))
                    * Fraction(float(wv[j, kk])) * Fraction(float(swr[j, kk // 128])))
        out.append(acc)
    return out


def test_fp8_forward_brute_force_ragged():
    rng = np.random.default_rng(7)
    m, k, n, e = 9, 320, 4, 3          # k: 2 full blocks and a partial third
    offs = np.array([3, 3, 7], dtype=np.int32)   # expert 1 empty, rows 7, 8 unused
    g = (k + 127) // 128
    x = rand_codes(rng, (m, k))
    w = rand_codes(rng, (e, n, k))
    sx = rand_pow2(rng, (m, g))
    sw = rand_pow2(rng, (e, n, g))
    res = oracle.fp8_forward(x, sx, w, sw, offs)
    owner = [0, 0, 0, 2, 2, 2, 2, None, None]
    for i in range(m):
        if owner[i] is None:
            assert res.status[i] == 0 and np.all(np.isnan(res.value[i]))
            continue
        assert res.status[i] == 1
        ex = exact_row(x[i], sx[i], w[owner[i]], sw[owner[i]])
        for j in range(n):
            bound = 2.0 ** -52 * k * res.sabs[i, j]
            assert abs(Fraction(res.value[i, j]) - ex[j]) <= Fraction(bound)
            assert res.sabs[i, j] >= abs(float(ex[j])) * (1 - 1e-12)


def test_fp8_forward_block_index():
    """A scale of k-block 1 multiplies exactly the products with k in
    [128, 256): doubling it three times adds 7x that partial sum."""
    rng = np.random.default_rng(8)
    m, k, n = 6, 384, 5
    offs = np.array([m], dtype=np.int32)
    x = rand_codes(rng, (m, k))
    w = rand_codes(rng, (1, n, k))
    sx = rand_pow2(rng, (m, 3))
    sw = rand_pow2(rng, (1, n, 3))
    base = oracle.fp8_forward(x, sx, w, sw, offs).value
    sx2 = sx.copy()
    sx2[:, 1] *= 8.0
    bumped = oracle.fp8_forward(x, sx2, w, sw, offs).value
    xd = torch_e4m3(x) * expand(sx, k)
    wd = torch_e4m3(w[0]) * expand(sw[0], k)
    partial = xd[:, 128:256] @ wd[:, 128:256].T
    np.testing.assert_allclose(bumped - base, 7.0 * partial, rtol=1e-12, atol=1e-300)
    # the weight scales' block index too
    sw2 = sw.copy()
    sw2[0, :, 2] *= 0.5
    halved = oracle.fp8_forward(x, sx, w, sw2, offs).value
    partial2 = xd[:, 256:] @ wd[:, 256:].T
    np.testing.assert_allclose(base - halved, 0.5 * partial2, rtol=1e-12, atol=1e-300)


def test_fp8_forward_matches_numpy_matmul():
    wl = synth.by_name("fp8_qwen3_gateup_small")
    t = synth.make_fp8_inputs(wl)
    x, sx = t["x8"].numpy(), t["sx"].numpy()
    w, sw = t["w8"].numpy(), t["sw"].numpy()
    offs = wl.offs
    rng = np.random.default_rng(9)
    rows = np.sort(rng.choice(wl.m, size=300, replace=False))
    res = oracle.fp8_forward(x, sx, w, sw, offs, rows=rows)
    ends = offs.astype(np.int64)
    xd = torch_e4m3(x[rows]) * expand(sx[rows], wl.k)
    for r, i in enumerate(rows):
        gi = int(np.searchsorted(ends, i, side="right"))
        wd = torch_e4m3(w[gi]) * expand(sw[gi], wl.k)
        ref = xd[r] @ wd.T
        np.testing.assert_allclose(res.value[r], ref, rtol=1e-11,
                                   atol=1e-13 * float(np.max(res.sabs[r])))


# --------------------------------------------------------------------------
# masked layout
# --------------------------------------------------------------------------

def test_fp8_masked_brute_force_and_inactive_rows():
    rng = np.random.default_rng(10)
    e, max_m, k, n = 3, 5, 256, 3
    mm = np.array([2, 0, 5], dtype=np.int32)
    x = rand_codes(rng, (e, max_m, k))
    w = rand_codes(rng, (e, n, k))
    sx = rand_pow2(rng, (e, max_m, 2))
    sw = rand_pow2(rng, (e, n, 2))
    for ex in range(e):                # inactive rows: NaN codes, garbage scales
        x[ex, mm[ex]:] = 0x7F
        sx[ex, mm[ex]:] = np.float32(0.3)
    res = oracle.fp8_masked_forward(x, sx, w, sw, mm)
    for ex in range(e):
        for r in range(max_m):
            flat = ex * max_m + r
            if r >= mm[ex]:
                assert res.status[flat] == 0
                continue
            exact = exact_row(x[ex, r], sx[ex, r], w[ex], sw[ex])
            for j in range(n):
                bound = 2.0 ** -52 * k * res.sabs[flat, j]
                assert abs(Fraction(res.value[flat, j]) - exact[j]) <= Fraction(bound)


def test_fp8_masked_equals_ragged_on_compacted_rows():
    wl = synth.by_name("fp8_masked_down_small")
    t = synth.make_fp8_inputs(wl)
    x, sx = t["x8"].numpy(), t["sx"].numpy()
    w, sw = t["w8"].numpy(), t["sw"].numpy()
    sizes = wl.group_sizes()
    masked = oracle.fp8_masked_forward(x, sx, w, sw, wl.masked_m)
    xc = np.concatenate([x[e, : sizes[e]] for e in range(wl.num_groups)])
    sxc = np.concatenate([sx[e, : sizes[e]] for e in range(wl.num_groups)])
    ragged = oracle.fp8_forward(xc, sxc, w, sw, np.cumsum(sizes).astype(np.int32))
    rows = np.concatenate([e * wl.m + np.arange(sizes[e]) for e in range(wl.num_groups)])
    assert np.array_equal(masked.value[rows], ragged.value)
    assert int(masked.status.sum()) == int(sizes.sum())


# --------------------------------------------------------------------------
# UE8M0 validity
# --------------------------------------------------------------------------

def test_ue8m0_violations_bit_patterns():
    good = np.array([1.0, 2.0 ** -5, 0.0, 2.0 ** 20, 2.0 ** -126], dtype=np.float32)
    bad = np.array([0.3, -1.0, 1.5, -0.0, np.nan], dtype=np.float32)
    assert oracle.ue8m0_violations(good) == 0
    assert oracle.ue8m0_violations(bad) == len(bad)
    both = np.stack([good, bad])
    active = np.array([[True] * 5, [True, False, True, False, False]])
    assert oracle.ue8m0_violations(both, active) == 2
    # the synthetic quantizer emits valid scales only
    t = synth.make_fp8_inputs(synth.by_name("fp8_masked_down_small"))
    sizes = synth.by_name("fp8_masked_down_small").group_sizes()
    act = np.arange(t["sx"].shape[1])[None, :, None] < sizes[:, None, None]
    act = np.broadcast_to(act, t["sx"].shape)
    assert oracle.ue8m0_violations(t["sx"].numpy(), act) == 0
    assert oracle.ue8m0_violations(t["sx"].numpy()) == int((~act).sum())
    assert oracle.ue8m0_violations(t["sw"].numpy()) == 0
