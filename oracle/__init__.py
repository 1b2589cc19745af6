"""fp64 CPU oracle for the bf16 grouped GEMM and its fp8 block-scaled
forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never touch it, and it shares no code with them: the arithmetic lives in
``oracle.c`` (plain per-group loops in fp64 with its own bf16 codec) and this
module only marshals numpy arrays into it.

What each function computes is stated, with the passages it follows, at the
top of ``oracle.c``; ``apply_alpha_beta`` adds the scaled, accumulating form
out = alpha * P + beta * C of every pass, combined in fp64 before the one
rounding.  Parity is pinned against exact rational brute force,
closed forms, the three-pass adjoint identity and numpy's float64 matmul in
``tests/test_oracle.py``, and the fp8 functions against torch's e4m3
decoding, exact rational brute force and numpy's matmul in
``tests/test_oracle_fp8.py``; no function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O3, OpenMP, no fast-math) into
    liboracle.so next to it."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-std=c11", "-O3", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int32
    sig = [P, P, P, I64, I64, I64, I32, P, I64, P, P, P]
    for name in ("oracle_forward", "oracle_dgrad", "oracle_wgrad",
                 "oracle_masked_forward", "oracle_masked_dgrad", "oracle_masked_wgrad"):
        f = getattr(lib, name)
        f.argtypes = sig
        f.restype = ctypes.c_int
    lib.oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    lib.oracle_round_bf16_array.argtypes = [P, I64, P]
    lib.oracle_round_bf16_array.restype = None
    lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_bf16.restype = ctypes.c_double
    for name in ("oracle_fp8_forward", "oracle_fp8_masked_forward"):
        f = getattr(lib, name)
        f.argtypes = [P, P, P, P, P, I64, I64, I64, I32, P, I64, P, P, P]
        f.restype = ctypes.c_int
    lib.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
    lib.oracle_decode_e4m3.restype = ctypes.c_double
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 operands are passed as uint16 bit arrays")
    return a


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def round_bf16(v) -> np.ndarray:
    """fp64 -> bf16 bits, round to nearest, ties to even (oracle_round_bf16,
    applied element-wise in C)."""
    lib = _load()
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib.oracle_round_bf16_array(_ptr(v), ctypes.c_int64(v.size), _ptr(out))
    return out


def round_bf16_scalar(v: float) -> int:
    return int(_load().oracle_round_bf16(float(v)))


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> float64, exact (bits << 16 is the fp32 pattern)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


class Result:
    """Oracle output: fp64 values, S = sum |a*b|, and which entries exist."""

    def __init__(self, value, sabs, status, index):
        self.value = value          # float64 [count, width]
        self.sabs = sabs            # float64 [count, width]
        self.status = status        # int32 [count]; 1 = computed
        self.index = index          # the rows / pairs that were asked for


def apply_alpha_beta(res: Result, alpha: float, beta: float, c_in=None) -> Result:
    """The scaled, accumulating form of a pass: out = alpha * P + beta * C,
    with P the grouped product the C oracle computed and C the output's prior
    contents, combined in fp64 before the single rounding to the output type
    -- fused accumulation, as opposed to adding an already rounded product
    (TransformerEngine PR #3542, "Changes": explicit alpha/beta and fused
    accumulation into fp32 outputs).  C is never read when beta == 0.

    c_in: the prior output rows the result covers, same shape as res.value,
    as bf16 bit patterns (uint16) or fp32 values.  S becomes |alpha| S +
    |beta C| (the magnitude that bounds the rounding error).  Entries the
    pass does not define (status 0) stay NaN."""
    alpha = float(alpha)
    beta = float(beta)
    value = alpha * res.value
    sabs = abs(alpha) * res.sabs
    if beta != 0.0:
        if c_in is None:
            raise ValueError("beta != 0 needs the prior output c_in")
        c = np.asarray(c_in)
        c = decode_bf16(c) if c.dtype == np.uint16 else c.astype(np.float64)
        assert c.shape == value.shape, (c.shape, value.shape)
        ok = (res.status == 1)[:, None]
        value = np.where(ok, value + beta * c, value)
        sabs = np.where(ok, sabs + abs(beta) * np.abs(c), sabs)
    return Result(value, sabs, res.status, res.index)


def _run(fname, a, b, sel_arr, count, width, call_args):
    lib = _load()
    value = np.full((count, width), np.nan, dtype=np.float64)
    sabs = np.full((count, width), np.nan, dtype=np.float64)
    status = np.zeros(count, dtype=np.int32)
    rc = getattr(lib, fname)(_ptr(a), _ptr(b), *call_args,
                             _ptr(sel_arr), ctypes.c_int64(0 if sel_arr is None else len(sel_arr)),
                             _ptr(value), _ptr(sabs), _ptr(status))
    if rc != 0:
        raise ValueError(f"{fname} rejected its arguments (code {rc})")
    return value, sabs, status


def forward(x, w, offs, rows=None, alpha=1.0, beta=0.0, c_in=None) -> Result:
    """Y rows of the ragged forward (oracle_forward).  x: uint16 [M,K];
    w: uint16 [E,K,N]; offs: int32 [E] end offsets; rows: row indices or
    None for all M rows; alpha, beta, c_in: see apply_alpha_beta."""
    x, w = _u16(x), _u16(w)
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    m, k = x.shape
    e, k2, n = w.shape
    assert k2 == k and offs.shape == (e,)
    sel = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    count = m if sel is None else len(sel)
    v, s, st = _run("oracle_forward", x, w, sel, count, n,
                    (_ptr(offs), ctypes.c_int64(m), ctypes.c_int64(k),
                     ctypes.c_int64(n), ctypes.c_int32(e)))
    res = Result(v, s, st, sel if sel is not None else np.arange(m))
    return apply_alpha_beta(res, alpha, beta, c_in)


def dgrad(dy, w, offs, rows=None, alpha=1.0, beta=0.0, c_in=None) -> Result:
    """dX rows of the ragged dgrad (oracle_dgrad).  dy: uint16 [M,N]."""
    dy, w = _u16(dy), _u16(w)
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    m, n = dy.shape
    e, k, n2 = w.shape
    assert n2 == n and offs.shape == (e,)
    sel = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    count = m if sel is None else len(sel)
    v, s, st = _run("oracle_dgrad", dy, w, sel, count, k,
                    (_ptr(offs), ctypes.c_int64(m), ctypes.c_int64(k),
                     ctypes.c_int64(n), ctypes.c_int32(e)))
    res = Result(v, s, st, sel if sel is not None else np.arange(m))
    return apply_alpha_beta(res, alpha, beta, c_in)


def wgrad(x, dy, offs, num_groups=None, pairs=None, alpha=1.0, beta=0.0, c_in=None) -> Result:
    """dW rows (expert g, k index kk) of the ragged wgrad (oracle_wgrad).
    pairs: int [P,2] of (g, kk), or None for all E*K rows in order."""
    x, dy = _u16(x), _u16(dy)
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    m, k = x.shape
    m2, n = dy.shape
    assert m2 == m
    e = len(offs) if num_groups is None else num_groups
    assert len(offs) == e
    sel = None if pairs is None else np.ascontiguousarray(pairs, dtype=np.int64).reshape(-1, 2)
    count = e * k if sel is None else len(sel)
    lib = _load()
    value = np.full((count, n), np.nan, dtype=np.float64)
    sabs = np.full((count, n), np.nan, dtype=np.float64)
    status = np.zeros(count, dtype=np.int32)
    rc = lib.oracle_wgrad(_ptr(x), _ptr(dy), _ptr(offs), ctypes.c_int64(m),
                          ctypes.c_int64(k), ctypes.c_int64(n), ctypes.c_int32(e),
                          _ptr(sel), ctypes.c_int64(0 if sel is None else len(sel)),
                          _ptr(value), _ptr(sabs), _ptr(status))
    if rc != 0:
        raise ValueError(f"oracle_wgrad rejected its arguments (code {rc})")
    idx = sel if sel is not None else np.stack(
        [np.repeat(np.arange(e), k), np.tile(np.arange(k), e)], axis=1)
    return apply_alpha_beta(Result(value, sabs, status, idx), alpha, beta, c_in)


def masked_forward(x, w, masked_m, rows=None, alpha=1.0, beta=0.0, c_in=None) -> Result:
    """Rows of the masked forward (oracle_masked_forward).  x: uint16
    [E, max_m, K]; rows: flat indices e*max_m + r, or None for all."""
    x, w = _u16(x), _u16(w)
    masked_m = np.ascontiguousarray(masked_m, dtype=np.int32)
    e, max_m, k = x.shape
    e2, k2, n = w.shape
    assert e2 == e and k2 == k and masked_m.shape == (e,)
    sel = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    count = e * max_m if sel is None else len(sel)
    v, s, st = _run("oracle_masked_forward", x, w, sel, count, n,
                    (_ptr(masked_m), ctypes.c_int64(max_m), ctypes.c_int64(k),
                     ctypes.c_int64(n), ctypes.c_int32(e)))
    res = Result(v, s, st, sel if sel is not None else np.arange(e * max_m))
    return apply_alpha_beta(res, alpha, beta, c_in)


def masked_dgrad(dy, w, masked_m, rows=None, alpha=1.0, beta=0.0, c_in=None) -> Result:
    """Rows of the masked dgrad (oracle_masked_dgrad).  dy: uint16
    [E, max_m, N]; w: uint16 [E, K, N]; rows: flat indices e*max_m + r, or
    None for all; the result rows are dX[e, r, :K]."""
    dy, w = _u16(dy), _u16(w)
    masked_m = np.ascontiguousarray(masked_m, dtype=np.int32)
    e, max_m, n = dy.shape
    e2, k, n2 = w.shape
    assert e2 == e and n2 == n and masked_m.shape == (e,)
    sel = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    count = e * max_m if sel is None else len(sel)
    v, s, st = _run("oracle_masked_dgrad", dy, w, sel, count, k,
                    (_ptr(masked_m), ctypes.c_int64(max_m), ctypes.c_int64(k),
                     ctypes.c_int64(n), ctypes.c_int32(e)))
    res = Result(v, s, st, sel if sel is not None else np.arange(e * max_m))
    return apply_alpha_beta(res, alpha, beta, c_in)


def masked_wgrad(x, dy, masked_m, pairs=None, alpha=1.0, beta=0.0, c_in=None) -> Result:
    """dW rows (expert e, k index kk) of the masked wgrad
    (oracle_masked_wgrad).  x: uint16 [E, max_m, K]; dy: uint16
    [E, max_m, N]; pairs: int [P, 2] of (e, kk), or None for all E*K rows."""
    x, dy = _u16(x), _u16(dy)
    masked_m = np.ascontiguousarray(masked_m, dtype=np.int32)
    e, max_m, k = x.shape
    e2, max_m2, n = dy.shape
    assert e2 == e and max_m2 == max_m and masked_m.shape == (e,)
    sel = None if pairs is None else np.ascontiguousarray(pairs, dtype=np.int64).reshape(-1, 2)
    count = e * k if sel is None else len(sel)
    lib = _load()
    value = np.full((count, n), np.nan, dtype=np.float64)
    sabs = np.full((count, n), np.nan, dtype=np.float64)
    status = np.zeros(count, dtype=np.int32)
    rc = lib.oracle_masked_wgrad(_ptr(x), _ptr(dy), _ptr(masked_m), ctypes.c_int64(max_m),
                                 ctypes.c_int64(k), ctypes.c_int64(n), ctypes.c_int32(e),
                                 _ptr(sel), ctypes.c_int64(0 if sel is None else len(sel)),
                                 _ptr(value), _ptr(sabs), _ptr(status))
    if rc != 0:
        raise ValueError(f"oracle_masked_wgrad rejected its arguments (code {rc})")
    idx = sel if sel is not None else np.stack(
        [np.repeat(np.arange(e), k), np.tile(np.arange(k), e)], axis=1)
    return apply_alpha_beta(Result(value, sabs, status, idx), alpha, beta, c_in)


def _silu_mul(gate: Result, up: Result) -> Result:
    """out = silu(G) * U with silu(z) = z / (1 + exp(-z)), on the fp64 gate
    and up products, before the one rounding (the activation step between
    the gate/up and down GEMMs: sglang PR #32385, "Cause"; fused into the
    gate/up epilogue).  S is replaced by a magnitude that bounds the
    propagated accumulation error: with d silu(z)/dz = s(z) (1 + z (1 - s(z)))
    and s the logistic function,
        S' = |silu'(G)| |U| S_G + |silu(G)| S_U + 4 |out|,
    the last term standing for the fp32 evaluation of silu * mul (the checks
    scale S by 2 L 2^-24, so it allows at least 8 fp32 ulps of the result)."""
    g, u = gate.value, up.value
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = sig * (1.0 + g * (1.0 - sig))
    value = silu * u
    sabs = np.abs(dsilu) * np.abs(u) * gate.sabs + np.abs(silu) * up.sabs + 4.0 * np.abs(value)
    return Result(value, sabs, gate.status, gate.index)


def forward_silu_mul(x, w13, offs, rows=None) -> Result:
    """Rows of the ragged gate/up forward with the SiLU-mul activation:
    A[i, c] = silu((X W13[g])[i, c]) * (X W13[g])[i, I + c], c < I, where
    w13 is [E, K, 2I] (gate columns first, then up).  Built on forward()."""
    w13 = _u16(w13)
    e, k, n2 = w13.shape
    assert n2 % 2 == 0
    i = n2 // 2
    gate = forward(x, np.ascontiguousarray(w13[:, :, :i]), offs, rows=rows)
    up = forward(x, np.ascontiguousarray(w13[:, :, i:]), offs, rows=rows)
    return _silu_mul(gate, up)


def masked_forward_silu_mul(x, w13, masked_m, rows=None) -> Result:
    """The masked layout's gate/up forward with the SiLU-mul activation
    (output [E, max_m, I], active rows only).  Built on masked_forward()."""
    w13 = _u16(w13)
    e, k, n2 = w13.shape
    assert n2 % 2 == 0
    i = n2 // 2
    gate = masked_forward(x, np.ascontiguousarray(w13[:, :, :i]), masked_m, rows=rows)
    up = masked_forward(x, np.ascontiguousarray(w13[:, :, i:]), masked_m, rows=rows)
    return _silu_mul(gate, up)


# ---- FP8 (e4m3) block-scaled forward ------------------------------------------

def decode_e4m3(b: int) -> float:
    """One e4m3 byte -> its value (oracle_decode_e4m3: OCP E4M3, bias 7,
    NaN only at S.1111.111, no infinities)."""
    return float(_load().oracle_decode_e4m3(int(b) & 0xFF))


def _u8(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        raise TypeError("fp8 operands are passed as uint8 byte arrays")
    return a


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def fp8_forward(x, sx, w, sw, offs, rows=None) -> Result:
    """Rows of the ragged fp8 block-scaled forward (oracle_fp8_forward):
    Y[i, n] = sum_k x[i, k] sx[i, k // 128] w[g, n, k] sw[g, n, k // 128].
    x: uint8 e4m3 [M, K]; sx: fp32 [M, ceil(K/128)]; w: uint8 e4m3
    [E, N, K]; sw: fp32 [E, N, ceil(K/128)]; offs: int32 [E] end offsets."""
    x, w = _u8(x), _u8(w)
    sx, sw = _f32(sx), _f32(sw)
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    m, k = x.shape
    e, n, k2 = w.shape
    kb = (k + 127) // 128
    assert k2 == k and offs.shape == (e,) and sx.shape == (m, kb) and sw.shape == (e, n, kb)
    sel = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    count = m if sel is None else len(sel)
    lib = _load()
    value = np.full((count, n), np.nan, dtype=np.float64)
    sabs = np.full((count, n), np.nan, dtype=np.float64)
    status = np.zeros(count, dtype=np.int32)
    rc = lib.oracle_fp8_forward(_ptr(x), _ptr(sx), _ptr(w), _ptr(sw), _ptr(offs),
                                ctypes.c_int64(m), ctypes.c_int64(k), ctypes.c_int64(n),
                                ctypes.c_int32(e), _ptr(sel),
                                ctypes.c_int64(0 if sel is None else len(sel)),
                                _ptr(value), _ptr(sabs), _ptr(status))
    if rc != 0:
        raise ValueError(f"oracle_fp8_forward rejected its arguments (code {rc})")
    return Result(value, sabs, status, sel if sel is not None else np.arange(m))


def fp8_masked_forward(x, sx, w, sw, masked_m, rows=None) -> Result:
    """Rows of the masked fp8 block-scaled forward
    (oracle_fp8_masked_forward).  x: uint8 [E, max_m, K]; sx: fp32
    [E, max_m, ceil(K/128)]; w, sw as in fp8_forward; rows: flat indices
    e*max_m + r, or None for all.  Inactive rows' values and scales are
    never read."""
    x, w = _u8(x), _u8(w)
    sx, sw = _f32(sx), _f32(sw)
    masked_m = np.ascontiguousarray(masked_m, dtype=np.int32)
    e, max_m, k = x.shape
    e2, n, k2 = w.shape
    kb = (k + 127) // 128
    assert e2 == e and k2 == k and masked_m.shape == (e,)
    assert sx.shape == (e, max_m, kb) and sw.shape == (e, n, kb)
    sel = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    count = e * max_m if sel is None else len(sel)
    lib = _load()
    value = np.full((count, n), np.nan, dtype=np.float64)
    sabs = np.full((count, n), np.nan, dtype=np.float64)
    status = np.zeros(count, dtype=np.int32)
    rc = lib.oracle_fp8_masked_forward(_ptr(x), _ptr(sx), _ptr(w), _ptr(sw), _ptr(masked_m),
                                       ctypes.c_int64(max_m), ctypes.c_int64(k),
                                       ctypes.c_int64(n), ctypes.c_int32(e), _ptr(sel),
                                       ctypes.c_int64(0 if sel is None else len(sel)),
                                       _ptr(value), _ptr(sabs), _ptr(status))
    if rc != 0:
        raise ValueError(f"oracle_fp8_masked_forward rejected its arguments (code {rc})")
    return Result(value, sabs, status, sel if sel is not None else np.arange(e * max_m))


def ue8m0_violations(scales, active=None) -> int:
    """Number of fp32 scales that are not UE8M0: whose sign or mantissa bits
    are set (sglang PR #32385, "Problem": the check masks an fp32 with
    0x807fffff and wants zero, which admits +0.0 and every positive power of
    two).  active: a boolean mask of the same shape selecting the entries
    that count (inactive rows are not validated, "Rejected alternatives"),
    or None for all."""
    bits = np.ascontiguousarray(scales, dtype=np.float32).view(np.uint32)
    bad = (bits & np.uint32(0x807FFFFF)) != 0
    if active is not None:
        bad = bad & np.asarray(active, dtype=bool)
    return int(bad.sum())


# ---- [E, N, K] weight layout --------------------------------------------------
# The same passes with W[g] stored as its transpose [n, k] and dW as
# [E, n, k] (TransformerEngine PR #3542, "Summary": TN / NN / NT forms).  A
# layout only: the weight is transposed (a copy, no arithmetic) and the
# [E, K, N] function computes.

def _t(w):
    return np.ascontiguousarray(np.swapaxes(_u16(w), 1, 2))


def forward_nk(x, w_nk, offs, rows=None) -> Result:
    """Y = X W[g]^T with w_nk uint16 [E, N, K]."""
    return forward(x, _t(w_nk), offs, rows=rows)


def dgrad_nk(dy, w_nk, offs, rows=None) -> Result:
    """dX = dY W[g] with w_nk uint16 [E, N, K] (dX rows are K wide)."""
    return dgrad(dy, _t(w_nk), offs, rows=rows)


def wgrad_nk(x, dy, offs, num_groups=None) -> Result:
    """dW[g] as [N, K]: the rows of the result are (g, n) pairs in order."""
    res = wgrad(x, dy, offs, num_groups=num_groups)
    e = len(offs) if num_groups is None else num_groups
    k = x.shape[1]
    n = dy.shape[1]
    v = np.ascontiguousarray(np.swapaxes(res.value.reshape(e, k, n), 1, 2)).reshape(e * n, k)
    sa = np.ascontiguousarray(np.swapaxes(res.sabs.reshape(e, k, n), 1, 2)).reshape(e * n, k)
    st = np.ones(e * n, dtype=np.int32)
    idx = np.stack([np.repeat(np.arange(e), n), np.tile(np.arange(n), e)], axis=1)
    return Result(v, sa, st, idx)


def masked_forward_nk(x, w_nk, masked_m, rows=None) -> Result:
    return masked_forward(x, _t(w_nk), masked_m, rows=rows)


# ---- grouped bias with a per-token factor ---------------------------------------
# y[i, :] = alpha P[i, :] + beta C[i, :] + s[i] bias[g, :] over the rows i of
# each expert g (TransformerEngine PR #3542, "Summary": grouped bias applied
# to the grouped GEMM's output; review finding "Bias scaling breaks
# capacity": s covers the logical rows only and capacity rows are kept), in
# fp64 before the one rounding.

def _clamped_ends(offs, m):
    ends = np.zeros(len(offs), dtype=np.int64)
    prev = 0
    for g, o in enumerate(np.asarray(offs, dtype=np.int64)):
        e = min(max(int(o), prev), m)
        ends[g] = e
        prev = e
    return ends


def _add_bias(res: Result, groups_of_rows, bias, scale_of_rows) -> Result:
    b = decode_bf16(np.asarray(bias, dtype=np.uint16))
    ok = res.status == 1
    add = np.zeros_like(res.value)
    add[ok] = scale_of_rows[ok, None] * b[groups_of_rows[ok]]
    value = np.where(ok[:, None], res.value + add, res.value)
    sabs = np.where(ok[:, None], res.sabs + np.abs(add), res.sabs)
    return Result(value, sabs, res.status, res.index)


def forward_bias(x, w, offs, bias, bias_scale=None, rows=None, alpha=1.0, beta=0.0, c_in=None) -> Result:
    """Rows of the ragged forward plus s[i] bias[g]: bias uint16 bf16 [E, N];
    bias_scale fp32 indexed by row (at least end(E-1) entries) or None for
    1.  Rows no expert owns keep status 0."""
    res = forward(x, w, offs, rows=rows, alpha=alpha, beta=beta, c_in=c_in)
    m = x.shape[0]
    ends = _clamped_ends(offs, m)
    idx = np.asarray(res.index, dtype=np.int64)
    grp = np.minimum(np.searchsorted(ends, idx, side="right"), len(ends) - 1)
    sc = np.ones(len(idx)) if bias_scale is None else np.zeros(len(idx))
    if bias_scale is not None:
        bs = np.asarray(bias_scale, dtype=np.float32).astype(np.float64)
        live = res.status == 1
        sc[live] = bs[idx[live]]
    return _add_bias(res, grp, bias, sc)


def masked_forward_bias(x, w, masked_m, bias, bias_scale=None, rows=None, alpha=1.0, beta=0.0,
                        c_in=None) -> Result:
    """The masked forward plus s[e * max_m + r] bias[e] on active rows."""
    res = masked_forward(x, w, masked_m, rows=rows, alpha=alpha, beta=beta, c_in=c_in)
    max_m = x.shape[1]
    idx = np.asarray(res.index, dtype=np.int64)
    grp = idx // max_m
    sc = np.ones(len(idx))
    if bias_scale is not None:
        bs = np.asarray(bias_scale, dtype=np.float32).astype(np.float64).reshape(-1)
        live = res.status == 1
        sc = np.zeros(len(idx))
        sc[live] = bs[idx[live]]
    return _add_bias(res, grp, bias, sc)


# ---- producing the grouped layout ------------------------------------------------
# PyTorch issue #152668, "Describe the bug": end offsets come from a
# permute-indices step that rounds each expert's token count up to
# min_alignment_m and (its fix) pads empty experts; TransformerEngine PR
# #3224: per-expert counts (m_splits) on the device.  Integer work, written
# out from those definitions: pad(c) = c rounded up to a multiple of align,
# at least align when pad_empty.

def pad_count(c: int, align: int, pad_empty: bool) -> int:
    c = max(int(c), 0)
    p = -(-c // align) * align
    if pad_empty and p < align:
        p = align
    return p


def offsets_from_splits(splits, align=1, pad_empty=False) -> np.ndarray:
    out, run = [], 0
    for c in splits:
        run += pad_count(c, align, pad_empty)
        out.append(run)
    return np.array(out, dtype=np.int64)


def route(expert_of_slot, num_groups, align=1, pad_empty=False):
    """Slots (token * topk + k) grouped by expert, each expert's slots in
    ascending order, followed by its padding rows (-1).  Returns offs,
    row_slot (length offs[-1]) and slot_row (-1 for a slot whose expert is
    outside [0, num_groups))."""
    ids = np.asarray(expert_of_slot, dtype=np.int64).reshape(-1)
    row_slot, slot_row = [], np.full(len(ids), -1, dtype=np.int64)
    offs = []
    for e in range(num_groups):
        mine = np.flatnonzero(ids == e).tolist()
        for s in mine:
            slot_row[s] = len(row_slot)
            row_slot.append(s)
        row_slot += [-1] * (pad_count(len(mine), align, pad_empty) - len(mine))
        offs.append(len(row_slot))
    return np.array(offs, dtype=np.int64), np.array(row_slot, dtype=np.int64), slot_row


def gather_rows(src, row_slot, topk):
    """Row r of the grouped layout: src[row_slot[r] // topk], zeros for -1."""
    src = np.asarray(src)
    out = np.zeros((len(row_slot),) + src.shape[1:], dtype=src.dtype)
    for r, s in enumerate(row_slot):
        if s >= 0:
            out[r] = src[s // topk]
    return out


def combine_rows(y_bits, slot_row, topk, weights=None) -> Result:
    """out[t] = sum_k w[t, k] y[slot_row[t topk + k]] in fp64 over the slots
    that were not dropped; y as bf16 bits.  S = sum |w y|."""
    y = decode_bf16(np.asarray(y_bits, dtype=np.uint16))
    slot_row = np.asarray(slot_row, dtype=np.int64).reshape(-1)
    tokens = len(slot_row) // topk
    w = np.ones((tokens, topk)) if weights is None else np.asarray(weights, dtype=np.float32).astype(np.float64)
    value = np.zeros((tokens, y.shape[1]))
    sabs = np.zeros((tokens, y.shape[1]))
    for t in range(tokens):
        for k in range(topk):
            r = slot_row[t * topk + k]
            if r >= 0:
                value[t] += w[t, k] * y[r]
                sabs[t] += np.abs(w[t, k] * y[r])
    return Result(value, sabs, np.ones(tokens, dtype=np.int32), np.arange(tokens))



def bias_grad(dy_bits, groups, bias_scale=None, masked=False) -> Result:
    """dbias[g, :] = sum_{i in g} s[i] dY[i, :] in fp64 (+0.0 for an empty
    expert); the backward of forward_bias's bias term.  Rows of the result
    are experts."""
    dy = decode_bf16(np.asarray(dy_bits, dtype=np.uint16))
    e = len(groups)
    if masked:
        max_m = dy.shape[1]
        dy = dy.reshape(-1, dy.shape[-1])
        spans = [(g * max_m, g * max_m + min(max(int(groups[g]), 0), max_m)) for g in range(e)]
    else:
        ends = _clamped_ends(groups, dy.shape[0])
        spans = [(0 if g == 0 else int(ends[g - 1]), int(ends[g])) for g in range(e)]
    s = None if bias_scale is None else np.asarray(bias_scale, dtype=np.float32).astype(np.float64).reshape(-1)
    value = np.zeros((e, dy.shape[1]))
    sabs = np.zeros((e, dy.shape[1]))
    for g, (a, b) in enumerate(spans):
        w = np.ones(b - a) if s is None else s[a:b]
        value[g] = (w[:, None] * dy[a:b]).sum(axis=0)
        sabs[g] = np.abs(w[:, None] * dy[a:b]).sum(axis=0)
    return Result(value, sabs, np.ones(e, dtype=np.int32), np.arange(e))


def bias_scale_grad(dy_bits, groups, bias_bits, masked=False) -> Result:
    """ds[i] = sum_n bias[g, n] dY[i, n] in fp64 for the rows an expert owns
    (status 1), rows of the result = flat rows."""
    dy = decode_bf16(np.asarray(dy_bits, dtype=np.uint16))
    b = decode_bf16(np.asarray(bias_bits, dtype=np.uint16))
    e = len(groups)
    if masked:
        max_m = dy.shape[1]
        dy = dy.reshape(-1, dy.shape[-1])
        owner = np.full(dy.shape[0], -1)
        for g in range(e):
            a = min(max(int(groups[g]), 0), max_m)
            owner[g * max_m: g * max_m + a] = g
    else:
        ends = _clamped_ends(groups, dy.shape[0])
        owner = np.full(dy.shape[0], -1)
        for g in range(e):
            owner[(0 if g == 0 else int(ends[g - 1])): int(ends[g])] = g
    ok = owner >= 0
    value = np.full((dy.shape[0], 1), np.nan)
    sabs = np.full((dy.shape[0], 1), np.nan)
    value[ok, 0] = (dy[ok] * b[owner[ok]]).sum(axis=1)
    sabs[ok, 0] = np.abs(dy[ok] * b[owner[ok]]).sum(axis=1)
    return Result(value, sabs, ok.astype(np.int32), np.arange(dy.shape[0]))
