"""Comparison of HIP results with the fp64 oracle (test infrastructure).

Tolerance (written here, used by every GPU parity test):

* bf16 outputs: an element passes if it is within 1 bf16 ulp of the oracle's
  value rounded to bf16 (distance on the ordered bit patterns, +0 == -0), or
  if |g - r| <= ulp_bf16(r) + 2 L 2^-24 S, where L is the reduction length and
  S = sum |a b| over the same terms (from the oracle).  The second clause is
  the fp32-accumulation error bound (any summation order: at most about
  L 2^-24 S, doubled for the MFMA's unspecified internal rounding) plus the
  final rounding; it matters only under cancellation (|r| << S), where one
  bf16 ulp of r is smaller than what any fp32 accumulation can promise.
* fp32 outputs: |g - r| <= 1e-2 max(1, |r|) and, tighter,
  |g - r| <= 2 L 2^-24 S + ulp_f32(r).
* the fp8 (e4m3) block-scaled forward (check_fp8): |g - r| <= ulp_out(r) +
  (2^-12 + K 2^-26) S, for either output type (bf16 also passes within 1
  ulp).  The scaled fp8 MFMA sums each run of 64 products with about 13
  significant bits before adding it into the fp32 accumulator: measured on
  MI355X over 32768 random dot products, |err| <= 2^-12.2 S_run for
  wide-range codes and <= 2^-14.5 S_run for Gaussian-quantized data, plus
  about 2^-21 of the accumulator per addition.  Summed over the K / 64 runs
  that gives the bound above (2^-12 S, and K / 64 * 2^-20 S for the
  accumulator term).
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
    bound = ulp_bf16(ref) + 2.0 * L * 2.0 ** -24 * sabs
    err = np.abs(g - ref)
    ok2 = err <= bound
    ok = ok1 | ok2
    if not np.all(ok):
        idx = np.argwhere(~ok)
        first = tuple(idx[0])
        raise AssertionError(
            f"{what}: {len(idx)} of {ok.size} bf16 elements out of tolerance; first at {first}: "
            f"got {g[first]!r} (0x{int(got_bits[first]):04x}) want {ref[first]!r} "
            f"(0x{int(ref_bits[first]):04x}), S={sabs[first]!r}, L={L}")
    if report is not None:
        report.n += ok.size
        report.exact += int(np.sum(dist == 0))
        report.within1 += int(np.sum(ok1))
        report.by_bound += int(np.sum(ok2 & ~ok1))
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


FP8_RUN_REL = 2.0 ** -12     # per-MFMA error of the fp8 dot product, relative to its S


def check_fp8(got, ref, sabs, K, what="", report: Report | None = None):
    """The fp8 forward's tolerance: ulp_out(r) + (2^-12 + K 2^-26) S."""
    ref = np.asarray(ref, dtype=np.float64)
    sabs = np.asarray(sabs, dtype=np.float64)
    tau = FP8_RUN_REL + K * 2.0 ** -26
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
        ok = np.abs(g - ref) <= bound
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
