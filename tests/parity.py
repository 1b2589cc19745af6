"""Comparison of HIP results with the fp64 oracle (test infrastructure).

Tolerance (written here, used by every GPU parity test):

* bf16 outputs: an element passes if it is within 1 bf16 ulp of the oracle's
  value rounded to bf16 (distance on the ordered bit patterns, +0 == -0).
  Under cancellation only, it may instead satisfy
  |g - r| <= ulp_bf16(r) + 2 L 2^-24 S, where L is the reduction length and
  S = sum |a b| over the same terms (from the oracle).  That second clause
  is the fp32-accumulation error bound (any summation order: at most about
  L 2^-24 S, doubled for the MFMA's unspecified internal rounding) plus the
  final rounding.  "Under cancellation" means |r| < 2^9 * 2 L 2^-24 S: where
  |r| is larger, that bound is at most half a bf16 ulp of r (2^-9 |r| <=
  ulp_bf16(r) / 2), so any fp32-accumulating kernel lands within 1 ulp and
  the element must.  At most 0.1 % of a check's elements (never more than
  one in a check of under 1000) may pass by the second clause alone: a
  kernel that lost accumulation precision (partial sums in bf16, say) would
  push far more elements past 1 ulp, and this fraction catches it.
* fp32 outputs: |g - r| <= 1e-2 max(1, |r|) and, tighter,
  |g - r| <= 2 L 2^-24 S + ulp_f32(r).
* the fp8 (e4m3) block-scaled forward (check_fp8): |g - r| <= ulp_out(r) +
  (2^-12 + K 2^-26) S (bf16 also passes within 1 ulp), and for fp32 outputs
  also |g - r| <= 1e-2 max(1, |r|).  The pages fix no precision for this
  path; the allowance is the worst case of a stated model of a block-scaled
  matrix unit (fp8_model_bound): the products of one 64-deep instruction are
  summed with at least 12 significant bits relative to their own magnitude
  sum (error <= 2^-12 S_run, truncation), and each instruction's result is
  added into the accumulator with at least 20 bits (error <= 2^-20 of the
  running sum, which is <= S).  Over the K / 64 instructions: 2^-12 S +
  (K / 64) 2^-20 S.  tests/test_parity_tolerance.py checks on the CPU that
  this check admits an emulation of that model at its worst and rejects one
  that sums in bf16.
"""
from __future__ import annotations

import numpy as np

import oracle


def dec_bf16(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ordered_bf16(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_bf16(r: np.ndarray) -> np.ndarray:
    a = np.abs(r)
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -126)
    return np.ldexp(1.0, e - 7)


def ulp_f32(r: np.ndarray) -> np.ndarray:
    a = np.abs(r).astype(np.float32)
    return np.abs(np.spacing(a).astype(np.float64))


# Largest share of a check's bf16 elements that may pass only by the
# cancellation clause (beyond 1 ulp of the rounded oracle value).
BOUND_FRACTION = 1e-3


class Report:
    def __init__(self):
        self.n = 0
        self.exact = 0
        self.within1 = 0
        self.by_bound = 0
        self.max_ulp = 0
        self.max_ratio = 0.0

    def __repr__(self):
        return (f"Report(n={self.n}, exact={self.exact}, within1ulp={self.within1}, "
                f"bound_only={self.by_bound}, max_ulp={self.max_ulp}, max_ratio={self.max_ratio:.3g})")


def check_bf16(got_bits, ref, sabs, L, what="", report: Report | None = None):
    got_bits = np.asarray(got_bits, dtype=np.uint16)
    ref = np.asarray(ref, dtype=np.float64)
    sabs = np.asarray(sabs, dtype=np.float64)
    assert got_bits.shape == ref.shape, (got_bits.shape, ref.shape)
    ref_bits = oracle.round_bf16(ref)
    dist = np.abs(ordered_bf16(got_bits) - ordered_bf16(ref_bits))
    ok1 = dist <= 1
    g = dec_bf16(got_bits)
    acc_bound = 2.0 * L * 2.0 ** -24 * sabs
    cancelling = np.abs(ref) < 2.0 ** 9 * acc_bound
    err = np.abs(g - ref)
    ok2 = cancelling & (err <= ulp_bf16(ref) + acc_bound)
    ok = ok1 | ok2
    if not np.all(ok):
        idx = np.argwhere(~ok)
        first = tuple(idx[0])
        raise AssertionError(
            f"{what}: {len(idx)} of {ok.size} bf16 elements out of tolerance; first at {first}: "
            f"got {g[first]!r} (0x{int(got_bits[first]):04x}) want {ref[first]!r} "
            f"(0x{int(ref_bits[first]):04x}), S={sabs[first]!r}, L={L}, "
            f"cancelling={bool(cancelling[first])}")
    by_bound = int(np.sum(ok2 & ~ok1))
    allowed = max(1, int(BOUND_FRACTION * ok.size))
    if by_bound > allowed:
        worst = np.unravel_index(int(np.argmax(np.where(ok1, -1, dist))), dist.shape)
        raise AssertionError(
            f"{what}: {by_bound} of {ok.size} bf16 elements are more than 1 ulp off (allowed {allowed}, "
            f"{BOUND_FRACTION:.1%}); worst at {tuple(worst)}: {int(dist[worst])} ulp, got {g[worst]!r} "
            f"want {ref[worst]!r}, S={sabs[worst]!r}")
    if report is not None:
        report.n += ok.size
        report.exact += int(np.sum(dist == 0))
        report.within1 += int(np.sum(ok1))
        report.by_bound += by_bound
        report.max_ulp = max(report.max_ulp, int(dist.max()) if dist.size else 0)
    return ok


def check_f32(got, ref, sabs, L, what="", report: Report | None = None):
    got = np.asarray(got, dtype=np.float32).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    sabs = np.asarray(sabs, dtype=np.float64)
    assert got.shape == ref.shape
    err = np.abs(got - ref)
    loose = err <= 1e-2 * np.maximum(1.0, np.abs(ref))
    tight_bound = 2.0 * L * 2.0 ** -24 * sabs + ulp_f32(ref)
    tight = err <= tight_bound
    ok = loose & tight
    if not np.all(ok):
        idx = np.argwhere(~ok)
        first = tuple(idx[0])
        raise AssertionError(
            f"{what}: {len(idx)} of {ok.size} fp32 elements out of tolerance; first at {first}: "
            f"got {got[first]!r} want {ref[first]!r}, S={sabs[first]!r}, L={L}")
    if report is not None:
        report.n += ok.size
        report.exact += int(np.sum(got.astype(np.float32) == ref.astype(np.float32)))
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.where(tight_bound > 0, err / tight_bound, 0.0)
        report.max_ratio = max(report.max_ratio, float(np.max(ratio)) if ratio.size else 0.0)
    return ok


def check(got, ref, sabs, L, what="", report=None):
    """Dispatch on the output's numpy dtype (uint16 = bf16 bits, float32)."""
    if got.dtype == np.uint16:
        return check_bf16(got, ref, sabs, L, what, report)
    return check_f32(got, ref, sabs, L, what, report)


# The fp8 accumulation model (see the module docstring): significant bits of
# one 64-deep block-scaled instruction's sum, and of each addition into the
# accumulator.
FP8_RUN_BITS = 12
FP8_ACC_BITS = 20
FP8_RUN = 64


def fp8_model_bound(K):
    """tau with |error| <= tau S under the model: 2^-12 + (K / 64) 2^-20."""
    return 2.0 ** -FP8_RUN_BITS + (K / FP8_RUN) * 2.0 ** -FP8_ACC_BITS


def check_fp8(got, ref, sabs, K, what="", report: Report | None = None):
    """The fp8 forward's tolerance: ulp_out(r) + tau S with tau =
    fp8_model_bound(K); fp32 outputs also within 1e-2 max(1, |r|)."""
    ref = np.asarray(ref, dtype=np.float64)
    sabs = np.asarray(sabs, dtype=np.float64)
    tau = fp8_model_bound(K)
    if got.dtype == np.uint16:
        ref_bits = oracle.round_bf16(ref)
        dist = np.abs(ordered_bf16(got) - ordered_bf16(ref_bits))
        g = dec_bf16(got)
        bound = ulp_bf16(ref) + tau * sabs
        ok = (dist <= 1) | (np.abs(g - ref) <= bound)
    else:
        g = np.asarray(got, dtype=np.float32).astype(np.float64)
        dist = None
        bound = ulp_f32(ref) + tau * sabs
        ok = (np.abs(g - ref) <= bound) & (np.abs(g - ref) <= 1e-2 * np.maximum(1.0, np.abs(ref)))
    if not np.all(ok):
        idx = np.argwhere(~ok)
        first = tuple(idx[0])
        raise AssertionError(
            f"{what}: {len(idx)} of {ok.size} elements out of the fp8 tolerance; first at {first}: "
            f"got {g[first]!r} want {ref[first]!r}, S={sabs[first]!r}, K={K}")
    if report is not None:
        report.n += ok.size
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.where(bound > 0, np.abs(g - ref) / bound, 0.0)
        report.max_ratio = max(report.max_ratio, float(np.max(ratio)) if ratio.size else 0.0)
        if dist is not None:
            report.exact += int(np.sum(dist == 0))
            report.within1 += int(np.sum(dist <= 1))
            report.max_ulp = max(report.max_ulp, int(dist.max()) if dist.size else 0)
    return ok
