"""The parity tolerances themselves (tests/parity.py), on the CPU.

A tolerance is only useful if it admits what a correct kernel may do and
rejects what a broken one does.  These tests feed the checks emulated
results, computed here in numpy from the oracle's own inputs:

* bf16: an fp32-accumulating dot product (16-term blocks added into an fp32
  running sum, the MFMA's shape of work) passes, with almost every element
  within 1 ulp; the same sum kept in bf16 between blocks fails on the
  fraction of elements that need the cancellation clause; a single element
  2 ulp off where |r| is far from cancellation fails.
* fp8: the accumulation model the fp8 allowance is derived from (each
  64-deep instruction's sum with an error of 2^-12 of its magnitude sum,
  each addition into the accumulator with 2^-20 of the running sum), driven
  to its worst case with every error in the same direction, passes; the
  same data summed in bf16 fails.
"""
import numpy as np
import pytest

import oracle
from moe_grouped_gemm_ragged_amd import synth
from parity import (BOUND_FRACTION, check_bf16, check_f32, check_fp8, fp8_model_bound,
                    FP8_ACC_BITS, FP8_RUN, FP8_RUN_BITS, Report)


def _round_sig(v, bits):
    """Round to nearest with `bits` significant bits (numpy fp64)."""
    m, e = np.frexp(v)
    return np.ldexp(np.round(m * 2.0 ** bits), e - bits)


def _dense_case(seed, m=192, k=1024, n=96):
    rng = np.random.default_rng(seed)
    x = synth_bits(rng.standard_normal((m, k)))
    w = synth_bits(0.02 * rng.standard_normal((1, k, n)))
    ref = oracle.forward(x, w, np.array([m], dtype=np.int32))
    return x, w, ref


def synth_bits(v):
    """fp64 values -> bf16 bit patterns (the oracle's rounding)."""
    return oracle.round_bf16(np.asarray(v, dtype=np.float64))


def _blocked_sum(x, w, acc_round, block=16):
    """sum over k in blocks of `block` products; each block's dot product in
    fp64 (exact for bf16 operands at these sizes up to the last bits), then
    added into a running sum rounded by acc_round after every addition."""
    xd = oracle.decode_bf16(x)
    wd = oracle.decode_bf16(w[0])
    acc = np.zeros((x.shape[0], wd.shape[1]))
    for k0 in range(0, xd.shape[1], block):
        part = xd[:, k0:k0 + block] @ wd[k0:k0 + block]
        acc = acc_round(acc + acc_round(part))
    return acc


def test_bf16_fp32_accumulation_passes():
    x, w, ref = _dense_case(1)
    got = synth_bits(_blocked_sum(x, w, lambda v: v.astype(np.float32).astype(np.float64)))
    rep = Report()
    check_bf16(got, ref.value, ref.sabs, x.shape[1], "fp32 accumulation", rep)
    assert rep.by_bound <= BOUND_FRACTION * rep.n
    assert rep.within1 >= (1 - BOUND_FRACTION) * rep.n


def test_bf16_partial_sums_in_bf16_fail():
    x, w, ref = _dense_case(2)
    bf16 = lambda v: oracle.decode_bf16(synth_bits(v))   # noqa: E731
    got = synth_bits(_blocked_sum(x, w, bf16))
    with pytest.raises(AssertionError, match="more than 1 ulp off|out of tolerance"):
        check_bf16(got, ref.value, ref.sabs, x.shape[1], "bf16 accumulation")


def test_bf16_two_ulp_off_outside_cancellation_fails():
    x, w, ref = _dense_case(3)
    got = synth_bits(ref.value)
    r = np.abs(ref.value)
    band = 2.0 ** 9 * 2.0 * x.shape[1] * 2.0 ** -24 * ref.sabs
    i, j = np.argwhere(r > 2 * band)[0]          # far from cancellation
    b = int(got[i, j])
    got[i, j] = b + 2 if b & 0x7FFF < 0x7F00 else b - 2
    with pytest.raises(AssertionError, match="out of tolerance"):
        check_bf16(got, ref.value, ref.sabs, x.shape[1], "planted 2 ulp")


def test_f32_cap_holds_with_a_loose_bound():
    # an error inside 2 L 2^-24 S but beyond 1e-2 max(1, |r|) is rejected
    ref = np.array([[1e-3, 5.0]])
    sabs = np.array([[1e6, 1e6]])
    got = (ref + np.array([[0.02, 0.0]])).astype(np.float32)
    with pytest.raises(AssertionError):
        check_f32(got, ref, sabs, 4096, "cap")


# ---- fp8 ----------------------------------------------------------------------

def _fp8_case():
    wl = synth.custom_ragged("tol_fp8", [160], k=1024, n=64, seed=91)
    t = synth.make_fp8_inputs(wl)
    x, sx = t["x8"].numpy(), t["sx"].numpy()
    w, sw = t["w8"].numpy(), t["sw"].numpy()
    ref = oracle.fp8_forward(x, sx, w, sw, wl.offs)
    table = np.array([oracle.decode_e4m3(c) for c in range(256)])
    xd = table[x] * np.repeat(sx.astype(np.float64), 128, axis=1)[:, : wl.k]
    wd = table[w[0]] * np.repeat(sw[0].astype(np.float64), 128, axis=1)[:, : wl.k]
    return wl, xd, wd, ref


def _fp8_emulate(xd, wd, run_err, acc_err):
    """Runs of FP8_RUN products: each run's sum gets run_err(s, S_run), each
    addition into the accumulator acc_err(acc)."""
    acc = np.zeros((xd.shape[0], wd.shape[0]))
    for k0 in range(0, xd.shape[1], FP8_RUN):
        a, b = xd[:, k0:k0 + FP8_RUN], wd[:, k0:k0 + FP8_RUN]
        s = a @ b.T
        s_abs = np.abs(a) @ np.abs(b).T
        acc = acc_err(acc + run_err(s, s_abs))
    return acc


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_fp8_model_worst_case_passes(out):
    wl, xd, wd, ref = _fp8_case()
    sign = np.sign(ref.value)
    sign[sign == 0] = 1.0
    # every error at its model bound, all in the same direction as r
    acc = _fp8_emulate(xd, wd, lambda s, S: s + sign * 2.0 ** -FP8_RUN_BITS * S,
                       lambda v: v + sign * 2.0 ** -FP8_ACC_BITS * np.abs(v))
    assert np.all(np.abs(acc - ref.value) <= fp8_model_bound(wl.k) * ref.sabs * (1 + 1e-9))
    got = synth_bits(acc) if out == "bf16" else acc.astype(np.float32)
    check_fp8(got, ref.value, ref.sabs, wl.k, "fp8 model, worst case")


def test_fp8_model_rounding_passes():
    wl, xd, wd, ref = _fp8_case()
    acc = _fp8_emulate(xd, wd, lambda s, S: _round_sig(s, FP8_RUN_BITS),
                       lambda v: _round_sig(v, FP8_ACC_BITS))
    check_fp8(synth_bits(acc), ref.value, ref.sabs, wl.k, "fp8 model, rounded")


def test_fp8_bf16_accumulation_fails():
    wl, xd, wd, ref = _fp8_case()
    acc = _fp8_emulate(xd, wd, lambda s, S: _round_sig(s, 8), lambda v: _round_sig(v, 8))
    with pytest.raises(AssertionError, match="fp8 tolerance"):
        check_fp8(acc.astype(np.float32), ref.value, ref.sabs, wl.k, "fp8 in bf16")
