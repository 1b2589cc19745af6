"""ctypes binding of libgg.so (the C ABI in include/gg.h).

Argument marshalling only: shapes, dtypes and devices are checked, outputs
are allocated with ``torch.empty`` when the caller passes none (the library
itself allocates nothing), and the pointers plus the current HIP stream go to
the C entry point of the same name.  Every step of the computation runs in
the HIP kernels; there is no fallback: if the library is missing or a call
fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libgg.so")
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "gg.h")
_lib = None

GG_BF16 = 0
GG_F32 = 1

STATUS = {
    0: "GG_OK",
    1: "GG_ERR_NULL_PTR",
    2: "GG_ERR_BAD_DIM",
    3: "GG_ERR_ALIGNMENT",
    4: "GG_ERR_BAD_DTYPE",
    5: "GG_ERR_LIMIT",
    6: "GG_ERR_HIP",
}


class GGError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        super().__init__(f"{fn} failed: {self.status_name}: {message}")


def library_path() -> str:
    return _LIB_PATH


def header_path() -> str:
    return _HEADER


def load():
    """Load libgg.so (built in-tree by moe_grouped_gemm_ragged_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m moe_grouped_gemm_ragged_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int32
    sig = [P, P, P, P, ctypes.c_int, I64, I64, I64, I32, P]
    for name in ("gg_forward", "gg_dgrad", "gg_wgrad", "gg_masked_forward", "gg_masked_dgrad",
                 "gg_masked_wgrad", "gg_forward_silu_mul", "gg_masked_forward_silu_mul",
                 "gg_forward_nk", "gg_dgrad_nk", "gg_wgrad_nk", "gg_masked_forward_nk"):
        f = getattr(lib, name)
        f.argtypes = sig
        f.restype = ctypes.c_int
    sig_ex = sig[:-1] + [ctypes.c_float, ctypes.c_float, P]
    for name in ("gg_forward_ex", "gg_dgrad_ex", "gg_wgrad_ex", "gg_masked_forward_ex",
                 "gg_masked_dgrad_ex", "gg_masked_wgrad_ex", "gg_forward_nk_ex", "gg_dgrad_nk_ex",
                 "gg_wgrad_nk_ex", "gg_masked_forward_nk_ex"):
        f = getattr(lib, name)
        f.argtypes = sig_ex
        f.restype = ctypes.c_int
    for name in ("gg_forward_bias", "gg_masked_forward_bias"):
        f = getattr(lib, name)
        f.argtypes = [P, P, P, P, P, P, ctypes.c_int, I64, I64, I64, I32, ctypes.c_float,
                      ctypes.c_float, P]
        f.restype = ctypes.c_int
    lib.gg_offsets_from_splits.argtypes = [P, I32, I32, ctypes.c_int, P, P]
    lib.gg_offsets_from_splits.restype = ctypes.c_int
    lib.gg_route_rows_bound.argtypes = [I64, I32, I32]
    lib.gg_route_rows_bound.restype = ctypes.c_int64
    lib.gg_route_workspace_bytes.argtypes = [I64, I32]
    lib.gg_route_workspace_bytes.restype = ctypes.c_int64
    lib.gg_route.argtypes = [P, I64, I32, I32, ctypes.c_int, P, P, I64, P, P, P]
    lib.gg_route.restype = ctypes.c_int
    lib.gg_route_noalloc.argtypes = [P, I64, I32, I32, ctypes.c_int, P, P, I64, P, P]
    lib.gg_route_noalloc.restype = ctypes.c_int
    lib.gg_gather_rows.argtypes = [P, I64, I64, P, I32, P, I32, I64, P, P]
    lib.gg_gather_rows.restype = ctypes.c_int
    lib.gg_combine_rows.argtypes = [P, I64, P, P, I32, I64, I64, P, ctypes.c_int, P]
    lib.gg_combine_rows.restype = ctypes.c_int
    for name in ("gg_bias_grad", "gg_masked_bias_grad", "gg_bias_scale_grad", "gg_masked_bias_scale_grad"):
        f = getattr(lib, name)
        f.argtypes = [P, P, P, P, I64, I64, I32, P]
        f.restype = ctypes.c_int
    lib.gg_fp8_scale_bytes.argtypes = [ctypes.c_int, I64, I64, I32]
    lib.gg_fp8_scale_bytes.restype = ctypes.c_int64
    lib.gg_fp8_pack_scales.argtypes = [ctypes.c_int, P, ctypes.c_int, I64, P, I64, I64, I32, P, P, P]
    lib.gg_fp8_pack_scales.restype = ctypes.c_int
    for name in ("gg_fp8_forward", "gg_fp8_masked_forward"):
        f = getattr(lib, name)
        f.argtypes = [P, P, P, P, P, P, ctypes.c_int, I64, I64, I64, I32, P]
        f.restype = ctypes.c_int
    lib.gg_status_str.argtypes = [ctypes.c_int]
    lib.gg_status_str.restype = ctypes.c_char_p
    lib.gg_last_error.argtypes = []
    lib.gg_last_error.restype = ctypes.c_char_p
    lib.gg_version.argtypes = []
    lib.gg_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_symbols():
    """Names of the functions include/gg.h declares."""
    with open(_HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gg_[a-z_]+)\s*\(", text)))


def call_raw(name: str, *args) -> int:
    """Call a C entry point with raw integer pointers/sizes; returns the
    gg_status code."""
    return int(getattr(load(), name)(*args))


def last_error() -> str:
    return load().gg_last_error().decode()


# ---------------------------------------------------------------------------
# torch-level helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.bfloat16:
        return GG_BF16
    if dt == torch.float32:
        return GG_F32
    raise TypeError(f"unsupported output dtype {dt}; use torch.bfloat16 or torch.float32")


def _check(t, name, dtype, ndim, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(device) -> int:
    torch = _torch()
    return int(torch.cuda.current_stream(device).cuda_stream)


def _invoke(name, a, b, groups, out, out_code, m, k, n, e, device, alpha=1.0, beta=0.0):
    """Calls the plain entry point, or its *_ex form when alpha != 1 or
    beta != 0."""
    if float(alpha) == 1.0 and float(beta) == 0.0:
        rc = call_raw(name, a.data_ptr(), b.data_ptr(), groups.data_ptr(), out.data_ptr(), out_code,
                      int(m), int(k), int(n), int(e), _stream_handle(device))
    else:
        name = name + "_ex"
        rc = call_raw(name, a.data_ptr(), b.data_ptr(), groups.data_ptr(), out.data_ptr(), out_code,
                      int(m), int(k), int(n), int(e), float(alpha), float(beta), _stream_handle(device))
    if rc != 0:
        raise GGError(name, rc, last_error())


def _need_out(out, beta):
    if float(beta) != 0.0 and out is None:
        raise ValueError("beta != 0 accumulates into `out`, which must be given")


def forward(x, w, offs, out: Optional["torch.Tensor"] = None, out_dtype=None, alpha=1.0, beta=0.0):
    """Y[rows of g] = X[rows of g] . W[g] (gg_forward).  x: bf16 [m,k];
    w: bf16 [E,k,n]; offs: int32 [E] cumulative end offsets on the device.
    Rows of ``out`` at or past offs[-1] are left untouched.  With alpha /
    beta, the written rows become alpha * product + beta * out
    (gg_forward_ex)."""
    torch = _torch()
    _need_out(out, beta)
    dev = x.device
    _check(x, "x", torch.bfloat16, 2, dev)
    _check(w, "w", torch.bfloat16, 3, dev)
    _check(offs, "offs", torch.int32, 1, dev)
    m, k = x.shape
    e, k2, n = w.shape
    if k2 != k or offs.shape[0] != e:
        raise ValueError("shape mismatch between x, w and offs")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype or torch.bfloat16, device=dev)
    _check(out, "out", out.dtype, 2, dev)
    if tuple(out.shape) != (m, n):
        raise ValueError(f"out must be [{m}, {n}]")
    _invoke("gg_forward", x, w, offs, out, _dtype_code(out.dtype), m, k, n, e, dev, alpha, beta)
    return out


def dgrad(dy, w, offs, out=None, out_dtype=None, alpha=1.0, beta=0.0):
    """dX[rows of g] = dY[rows of g] . W[g]^T (gg_dgrad).  dy: bf16 [m,n].
    alpha / beta as in forward (gg_dgrad_ex)."""
    torch = _torch()
    _need_out(out, beta)
    dev = dy.device
    _check(dy, "dy", torch.bfloat16, 2, dev)
    _check(w, "w", torch.bfloat16, 3, dev)
    _check(offs, "offs", torch.int32, 1, dev)
    m, n = dy.shape
    e, k, n2 = w.shape
    if n2 != n or offs.shape[0] != e:
        raise ValueError("shape mismatch between dy, w and offs")
    if out is None:
        out = torch.empty((m, k), dtype=out_dtype or torch.bfloat16, device=dev)
    _check(out, "out", out.dtype, 2, dev)
    if tuple(out.shape) != (m, k):
        raise ValueError(f"out must be [{m}, {k}]")
    _invoke("gg_dgrad", dy, w, offs, out, _dtype_code(out.dtype), m, k, n, e, dev, alpha, beta)
    return out


def wgrad(x, dy, offs, out=None, out_dtype=None, alpha=1.0, beta=0.0):
    """dW[g] = X[rows of g]^T . dY[rows of g] for every expert (gg_wgrad);
    all of ``out`` [E,k,n] is written, empty experts get +0.0.  beta = 1
    accumulates into ``out`` (e.g. an fp32 main-grad; gg_wgrad_ex)."""
    torch = _torch()
    _need_out(out, beta)
    dev = x.device
    _check(x, "x", torch.bfloat16, 2, dev)
    _check(dy, "dy", torch.bfloat16, 2, dev)
    _check(offs, "offs", torch.int32, 1, dev)
    m, k = x.shape
    m2, n = dy.shape
    e = offs.shape[0]
    if m2 != m:
        raise ValueError("x and dy must have the same number of rows")
    if out is None:
        out = torch.empty((e, k, n), dtype=out_dtype or torch.float32, device=dev)
    _check(out, "out", out.dtype, 3, dev)
    if tuple(out.shape) != (e, k, n):
        raise ValueError(f"out must be [{e}, {k}, {n}]")
    _invoke("gg_wgrad", x, dy, offs, out, _dtype_code(out.dtype), m, k, n, e, dev, alpha, beta)
    return out


def masked_forward(x, w, masked_m, out=None, out_dtype=None, alpha=1.0, beta=0.0):
    """Y[e, r] = X[e, r] . W[e] for r < masked_m[e] (gg_masked_forward).
    x: bf16 [E, max_m, k]; inactive rows are neither read nor written.
    alpha / beta as in forward (gg_masked_forward_ex)."""
    torch = _torch()
    _need_out(out, beta)
    dev = x.device
    _check(x, "x", torch.bfloat16, 3, dev)
    _check(w, "w", torch.bfloat16, 3, dev)
    _check(masked_m, "masked_m", torch.int32, 1, dev)
    e, max_m, k = x.shape
    e2, k2, n = w.shape
    if e2 != e or k2 != k or masked_m.shape[0] != e:
        raise ValueError("shape mismatch between x, w and masked_m")
    if out is None:
        out = torch.empty((e, max_m, n), dtype=out_dtype or torch.bfloat16, device=dev)
    _check(out, "out", out.dtype, 3, dev)
    if tuple(out.shape) != (e, max_m, n):
        raise ValueError(f"out must be [{e}, {max_m}, {n}]")
    _invoke("gg_masked_forward", x, w, masked_m, out, _dtype_code(out.dtype), max_m, k, n, e, dev,
            alpha, beta)
    return out


def masked_dgrad(dy, w, masked_m, out=None, out_dtype=None, alpha=1.0, beta=0.0):
    """dX[e, r] = dY[e, r] . W[e]^T for r < masked_m[e] (gg_masked_dgrad).
    dy: bf16 [E, max_m, n]; w: bf16 [E, k, n]; only active rows of ``out``
    [E, max_m, k] are written."""
    torch = _torch()
    _need_out(out, beta)
    dev = dy.device
    _check(dy, "dy", torch.bfloat16, 3, dev)
    _check(w, "w", torch.bfloat16, 3, dev)
    _check(masked_m, "masked_m", torch.int32, 1, dev)
    e, max_m, n = dy.shape
    e2, k, n2 = w.shape
    if e2 != e or n2 != n or masked_m.shape[0] != e:
        raise ValueError("shape mismatch between dy, w and masked_m")
    if out is None:
        out = torch.empty((e, max_m, k), dtype=out_dtype or torch.bfloat16, device=dev)
    _check(out, "out", out.dtype, 3, dev)
    if tuple(out.shape) != (e, max_m, k):
        raise ValueError(f"out must be [{e}, {max_m}, {k}]")
    _invoke("gg_masked_dgrad", dy, w, masked_m, out, _dtype_code(out.dtype), max_m, k, n, e, dev,
            alpha, beta)
    return out


def masked_wgrad(x, dy, masked_m, out=None, out_dtype=None, alpha=1.0, beta=0.0):
    """dW[e] = X[e, :a]^T . dY[e, :a], a = masked_m[e] clamped, for every
    expert (gg_masked_wgrad); all of ``out`` [E, k, n] is written."""
    torch = _torch()
    _need_out(out, beta)
    dev = x.device
    _check(x, "x", torch.bfloat16, 3, dev)
    _check(dy, "dy", torch.bfloat16, 3, dev)
    _check(masked_m, "masked_m", torch.int32, 1, dev)
    e, max_m, k = x.shape
    e2, max_m2, n = dy.shape
    if e2 != e or max_m2 != max_m or masked_m.shape[0] != e:
        raise ValueError("shape mismatch between x, dy and masked_m")
    if out is None:
        out = torch.empty((e, k, n), dtype=out_dtype or torch.float32, device=dev)
    _check(out, "out", out.dtype, 3, dev)
    if tuple(out.shape) != (e, k, n):
        raise ValueError(f"out must be [{e}, {k}, {n}]")
    _invoke("gg_masked_wgrad", x, dy, masked_m, out, _dtype_code(out.dtype), max_m, k, n, e, dev,
            alpha, beta)
    return out


def forward_silu_mul(x, w13, offs, out=None, out_dtype=None):
    """out[i, c] = silu(G)[i, c] * U[i, c] with [G | U] = X[rows of g] .
    W13[g] (gg_forward_silu_mul).  x: bf16 [m, k]; w13: bf16 [E, k, 2I]
    (gate columns, then up); returns [m, I]."""
    torch = _torch()
    dev = x.device
    _check(x, "x", torch.bfloat16, 2, dev)
    _check(w13, "w13", torch.bfloat16, 3, dev)
    _check(offs, "offs", torch.int32, 1, dev)
    m, k = x.shape
    e, k2, n = w13.shape
    if k2 != k or offs.shape[0] != e or n % 2:
        raise ValueError("shape mismatch between x, w13 and offs")
    if out is None:
        out = torch.empty((m, n // 2), dtype=out_dtype or torch.bfloat16, device=dev)
    _check(out, "out", out.dtype, 2, dev)
    if tuple(out.shape) != (m, n // 2):
        raise ValueError(f"out must be [{m}, {n // 2}]")
    _invoke("gg_forward_silu_mul", x, w13, offs, out, _dtype_code(out.dtype), m, k, n, e, dev)
    return out


def masked_forward_silu_mul(x, w13, masked_m, out=None, out_dtype=None):
    """The masked layout's gate/up forward with the SiLU-mul activation
    (gg_masked_forward_silu_mul): x bf16 [E, max_m, k] -> [E, max_m, I]."""
    torch = _torch()
    dev = x.device
    _check(x, "x", torch.bfloat16, 3, dev)
    _check(w13, "w13", torch.bfloat16, 3, dev)
    _check(masked_m, "masked_m", torch.int32, 1, dev)
    e, max_m, k = x.shape
    e2, k2, n = w13.shape
    if e2 != e or k2 != k or masked_m.shape[0] != e or n % 2:
        raise ValueError("shape mismatch between x, w13 and masked_m")
    if out is None:
        out = torch.empty((e, max_m, n // 2), dtype=out_dtype or torch.bfloat16, device=dev)
    _check(out, "out", out.dtype, 3, dev)
    if tuple(out.shape) != (e, max_m, n // 2):
        raise ValueError(f"out must be [{e}, {max_m}, {n // 2}]")
    _invoke("gg_masked_forward_silu_mul", x, w13, masked_m, out, _dtype_code(out.dtype), max_m, k, n,
            e, dev)
    return out


# ---------------------------------------------------------------------------
# producing the grouped layout
# ---------------------------------------------------------------------------

def _raise(name, rc):
    if rc != 0:
        raise GGError(name, rc, last_error())


def offsets_from_splits(m_splits, min_alignment=1, pad_empty=False, out=None):
    """int32 end offsets from int64 per-expert row counts on the device
    (gg_offsets_from_splits), each count padded to min_alignment."""
    torch = _torch()
    dev = m_splits.device
    _check(m_splits, "m_splits", torch.int64, 1, dev)
    e = m_splits.shape[0]
    if out is None:
        out = torch.empty(e, dtype=torch.int32, device=dev)
    _check(out, "out", torch.int32, 1, dev)
    _raise("gg_offsets_from_splits", call_raw("gg_offsets_from_splits", m_splits.data_ptr(), int(e),
                                              int(min_alignment), 1 if pad_empty else 0, out.data_ptr(),
                                              _stream_handle(dev)))
    return out


def route_rows_bound(slots, num_groups, min_alignment=1) -> int:
    v = int(load().gg_route_rows_bound(int(slots), int(num_groups), int(min_alignment)))
    if v < 0:
        raise ValueError("invalid arguments for gg_route_rows_bound")
    return v


def route(expert_of_slot, num_groups, min_alignment=1, pad_empty=False, rows_cap=None):
    """Token slots -> grouped layout (gg_route).  expert_of_slot: int32
    [tokens, topk] (or flat) expert ids.  Returns (offs int32 [E], row_slot
    int32 [rows_cap], slot_row int32 [slots]); row_slot past offs[-1] is
    uninitialised."""
    torch = _torch()
    dev = expert_of_slot.device
    if expert_of_slot.dtype != torch.int32 or not expert_of_slot.is_contiguous():
        raise TypeError("expert_of_slot must be a contiguous int32 tensor")
    slots = expert_of_slot.numel()
    cap = route_rows_bound(slots, num_groups, min_alignment) if rows_cap is None else int(rows_cap)
    offs = torch.empty(num_groups, dtype=torch.int32, device=dev)
    row_slot = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    slot_row = torch.empty(max(slots, 1), dtype=torch.int32, device=dev)
    ws = torch.empty(int(load().gg_route_workspace_bytes(slots, num_groups)), dtype=torch.uint8, device=dev)
    _raise("gg_route", call_raw("gg_route", expert_of_slot.data_ptr(), int(slots), int(num_groups),
                                int(min_alignment), 1 if pad_empty else 0, offs.data_ptr(),
                                row_slot.data_ptr(), int(cap), slot_row.data_ptr(), ws.data_ptr(),
                                _stream_handle(dev)))
    return offs, row_slot[:cap], slot_row[:slots]


def gather_rows(src, row_slot, topk, offs, out=None):
    """Grouped rows from token rows (gg_gather_rows): src [tokens, ...]
    (any dtype, rows a multiple of 16 bytes); returns [len(row_slot), ...]."""
    torch = _torch()
    dev = src.device
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    tokens = src.shape[0]
    row_bytes = src[0].numel() * src.element_size() if tokens else src.shape[1:].numel() * src.element_size()
    rows_cap = row_slot.shape[0]
    if out is None:
        out = torch.empty((rows_cap, *src.shape[1:]), dtype=src.dtype, device=dev)
    _raise("gg_gather_rows", call_raw("gg_gather_rows", src.data_ptr(), int(tokens), int(row_bytes),
                                      row_slot.data_ptr(), int(topk), offs.data_ptr(), int(offs.shape[0]),
                                      int(rows_cap), out.data_ptr(), _stream_handle(dev)))
    return out


def combine_rows(y, slot_row, topk, weights=None, out=None, out_dtype=None):
    """out[t] = sum_k w[t, k] y[slot_row[t topk + k]] (gg_combine_rows): y
    bf16 [rows, n]; weights fp32 [tokens, topk] or None."""
    torch = _torch()
    dev = y.device
    _check(y, "y", torch.bfloat16, 2, dev)
    rows_cap, n = y.shape
    slots = slot_row.numel()
    tokens = slots // topk
    if out is None:
        out = torch.empty((tokens, n), dtype=out_dtype or torch.bfloat16, device=dev)
    _raise("gg_combine_rows", call_raw("gg_combine_rows", y.data_ptr(), int(n), slot_row.data_ptr(),
                                       None if weights is None else weights.data_ptr(), int(topk),
                                       int(tokens), int(rows_cap), out.data_ptr(), _dtype_code(out.dtype),
                                       _stream_handle(dev)))
    return out


# ---------------------------------------------------------------------------
# grouped bias with a per-token factor
# ---------------------------------------------------------------------------

def _bias_call(name, x, w, groups, bias, bias_scale, out, m, k, n, e, dev, alpha, beta):
    torch = _torch()
    _check(bias, "bias", torch.bfloat16, 2, dev)
    if tuple(bias.shape) != (e, n):
        raise ValueError(f"bias must be [{e}, {n}]")
    if bias_scale is not None:
        if bias_scale.dtype != torch.float32 or bias_scale.device != dev or not bias_scale.is_contiguous():
            raise TypeError("bias_scale must be a contiguous float32 tensor on the device")
    rc = call_raw(name, x.data_ptr(), w.data_ptr(), groups.data_ptr(), bias.data_ptr(),
                  None if bias_scale is None else bias_scale.data_ptr(), out.data_ptr(),
                  _dtype_code(out.dtype), int(m), int(k), int(n), int(e), float(alpha), float(beta),
                  _stream_handle(dev))
    if rc != 0:
        raise GGError(name, rc, last_error())


def forward_bias(x, w, offs, bias, bias_scale=None, out=None, out_dtype=None, alpha=1.0, beta=0.0):
    """Y[i] = alpha X[i] W[g] + beta Y[i] + s[i] bias[g] on the rows of each
    expert (gg_forward_bias).  bias: bf16 [E, n]; bias_scale: fp32 with at
    least offs[-1] entries (the logical tokens), or None for 1."""
    torch = _torch()
    _need_out(out, beta)
    dev = x.device
    _check(x, "x", torch.bfloat16, 2, dev)
    _check(w, "w", torch.bfloat16, 3, dev)
    _check(offs, "offs", torch.int32, 1, dev)
    m, k = x.shape
    e, k2, n = w.shape
    if k2 != k or offs.shape[0] != e:
        raise ValueError("shape mismatch between x, w and offs")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype or torch.bfloat16, device=dev)
    _check(out, "out", out.dtype, 2, dev)
    if tuple(out.shape) != (m, n):
        raise ValueError(f"out must be [{m}, {n}]")
    _bias_call("gg_forward_bias", x, w, offs, bias, bias_scale, out, m, k, n, e, dev, alpha, beta)
    return out


def masked_forward_bias(x, w, masked_m, bias, bias_scale=None, out=None, out_dtype=None, alpha=1.0,
                        beta=0.0):
    """The masked forward plus s[e, r] bias[e] on active rows
    (gg_masked_forward_bias); bias_scale: fp32 [E, max_m] or None."""
    torch = _torch()
    _need_out(out, beta)
    dev = x.device
    _check(x, "x", torch.bfloat16, 3, dev)
    _check(w, "w", torch.bfloat16, 3, dev)
    _check(masked_m, "masked_m", torch.int32, 1, dev)
    e, max_m, k = x.shape
    e2, k2, n = w.shape
    if e2 != e or k2 != k or masked_m.shape[0] != e:
        raise ValueError("shape mismatch between x, w and masked_m")
    if out is None:
        out = torch.empty((e, max_m, n), dtype=out_dtype or torch.bfloat16, device=dev)
    _check(out, "out", out.dtype, 3, dev)
    if tuple(out.shape) != (e, max_m, n):
        raise ValueError(f"out must be [{e}, {max_m}, {n}]")
    _bias_call("gg_masked_forward_bias", x, w, masked_m, bias, bias_scale, out, max_m, k, n, e, dev,
               alpha, beta)
    return out


def bias_grad(dy, groups, bias_scale=None, masked=False, out=None):
    """dbias[g] = sum_{i in g} s[i] dY[i] (gg_bias_grad / gg_masked_bias_grad):
    dy bf16 [m, n] or [E, max_m, n]; returns fp32 [E, n]."""
    torch = _torch()
    dev = dy.device
    _check(dy, "dy", torch.bfloat16, 3 if masked else 2, dev)
    _check(groups, "groups", torch.int32, 1, dev)
    e = groups.shape[0]
    rows, n = (dy.shape[1], dy.shape[2]) if masked else (dy.shape[0], dy.shape[1])
    if out is None:
        out = torch.empty((e, n), dtype=torch.float32, device=dev)
    _check(out, "out", torch.float32, 2, dev)
    name = "gg_masked_bias_grad" if masked else "gg_bias_grad"
    _raise(name, call_raw(name, dy.data_ptr(), groups.data_ptr(),
                          None if bias_scale is None else bias_scale.data_ptr(), out.data_ptr(), int(rows),
                          int(n), int(e), _stream_handle(dev)))
    return out


def bias_scale_grad(dy, groups, bias, masked=False, out=None):
    """ds[i] = <bias[g], dY[i]> on the rows an expert owns
    (gg_bias_scale_grad / gg_masked_bias_scale_grad); returns fp32 [rows]
    (other entries as ``out`` held them; NaN when allocated here)."""
    torch = _torch()
    dev = dy.device
    _check(dy, "dy", torch.bfloat16, 3 if masked else 2, dev)
    _check(groups, "groups", torch.int32, 1, dev)
    _check(bias, "bias", torch.bfloat16, 2, dev)
    e = groups.shape[0]
    rows, n = (dy.shape[1], dy.shape[2]) if masked else (dy.shape[0], dy.shape[1])
    total = e * rows if masked else rows
    if out is None:
        out = torch.full((total,), float("nan"), dtype=torch.float32, device=dev)
    _check(out, "out", torch.float32, 1, dev)
    name = "gg_masked_bias_scale_grad" if masked else "gg_bias_scale_grad"
    _raise(name, call_raw(name, dy.data_ptr(), groups.data_ptr(), bias.data_ptr(), out.data_ptr(), int(rows),
                          int(n), int(e), _stream_handle(dev)))
    return out


# ---------------------------------------------------------------------------
# [E, N, K] weight layout
# ---------------------------------------------------------------------------

def forward_nk(x, w, offs, out=None, out_dtype=None, alpha=1.0, beta=0.0):
    """Y = X W[g]^T with W [E, n, k] (gg_forward_nk).  x: bf16 [m, k]."""
    torch = _torch()
    _need_out(out, beta)
    dev = x.device
    _check(x, "x", torch.bfloat16, 2, dev)
    _check(w, "w", torch.bfloat16, 3, dev)
    _check(offs, "offs", torch.int32, 1, dev)
    m, k = x.shape
    e, n, k2 = w.shape
    if k2 != k or offs.shape[0] != e:
        raise ValueError("shape mismatch between x, w and offs")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype or torch.bfloat16, device=dev)
    _check(out, "out", out.dtype, 2, dev)
    if tuple(out.shape) != (m, n):
        raise ValueError(f"out must be [{m}, {n}]")
    _invoke("gg_forward_nk", x, w, offs, out, _dtype_code(out.dtype), m, k, n, e, dev, alpha, beta)
    return out


def dgrad_nk(dy, w, offs, out=None, out_dtype=None, alpha=1.0, beta=0.0):
    """dX = dY W[g] with W [E, n, k] (gg_dgrad_nk).  dy: bf16 [m, n]."""
    torch = _torch()
    _need_out(out, beta)
    dev = dy.device
    _check(dy, "dy", torch.bfloat16, 2, dev)
    _check(w, "w", torch.bfloat16, 3, dev)
    _check(offs, "offs", torch.int32, 1, dev)
    m, n = dy.shape
    e, n2, k = w.shape
    if n2 != n or offs.shape[0] != e:
        raise ValueError("shape mismatch between dy, w and offs")
    if out is None:
        out = torch.empty((m, k), dtype=out_dtype or torch.bfloat16, device=dev)
    _check(out, "out", out.dtype, 2, dev)
    if tuple(out.shape) != (m, k):
        raise ValueError(f"out must be [{m}, {k}]")
    _invoke("gg_dgrad_nk", dy, w, offs, out, _dtype_code(out.dtype), m, k, n, e, dev, alpha, beta)
    return out


def wgrad_nk(x, dy, offs, out=None, out_dtype=None, alpha=1.0, beta=0.0):
    """dW[g] = dY[rows of g]^T X[rows of g], dW as [E, n, k] (gg_wgrad_nk)."""
    torch = _torch()
    _need_out(out, beta)
    dev = x.device
    _check(x, "x", torch.bfloat16, 2, dev)
    _check(dy, "dy", torch.bfloat16, 2, dev)
    _check(offs, "offs", torch.int32, 1, dev)
    m, k = x.shape
    m2, n = dy.shape
    e = offs.shape[0]
    if m2 != m:
        raise ValueError("x and dy must have the same rows")
    if out is None:
        out = torch.empty((e, n, k), dtype=out_dtype or torch.float32, device=dev)
    _check(out, "out", out.dtype, 3, dev)
    if tuple(out.shape) != (e, n, k):
        raise ValueError(f"out must be [{e}, {n}, {k}]")
    _invoke("gg_wgrad_nk", x, dy, offs, out, _dtype_code(out.dtype), m, k, n, e, dev, alpha, beta)
    return out


def masked_forward_nk(x, w, masked_m, out=None, out_dtype=None, alpha=1.0, beta=0.0):
    """The masked forward with W [E, n, k] (gg_masked_forward_nk)."""
    torch = _torch()
    _need_out(out, beta)
    dev = x.device
    _check(x, "x", torch.bfloat16, 3, dev)
    _check(w, "w", torch.bfloat16, 3, dev)
    _check(masked_m, "masked_m", torch.int32, 1, dev)
    e, max_m, k = x.shape
    e2, n, k2 = w.shape
    if e2 != e or k2 != k or masked_m.shape[0] != e:
        raise ValueError("shape mismatch between x, w and masked_m")
    if out is None:
        out = torch.empty((e, max_m, n), dtype=out_dtype or torch.bfloat16, device=dev)
    _check(out, "out", out.dtype, 3, dev)
    if tuple(out.shape) != (e, max_m, n):
        raise ValueError(f"out must be [{e}, {max_m}, {n}]")
    _invoke("gg_masked_forward_nk", x, w, masked_m, out, _dtype_code(out.dtype), max_m, k, n, e, dev,
            alpha, beta)
    return out


# ---------------------------------------------------------------------------
# fp8 (e4m3) block-scaled forward
# ---------------------------------------------------------------------------

GG_FP8_ACT_RAGGED = 0
GG_FP8_ACT_MASKED = 1
GG_FP8_WEIGHT = 2


def fp8_scale_bytes(layout: int, rows: int, k: int, num_groups: int) -> int:
    """Bytes of packed scales (gg_fp8_scale_bytes)."""
    v = int(load().gg_fp8_scale_bytes(int(layout), int(rows), int(k), int(num_groups)))
    if v < 0:
        raise ValueError("invalid arguments for gg_fp8_scale_bytes")
    return v


def fp8_pack_scales(layout: int, scales, groups, rows: int, k: int, num_groups: int,
                    out=None, bad_count=None):
    """Packed E8M0 scales of one operand (gg_fp8_pack_scales).  scales: fp32
    or uint8 (E8M0 bytes) with one scale per (row, k-block) in its last dim
    (rows flattened: [m, G], [E, max_m, G] or [E, n, G]; G may be padded);
    groups: the int32 end offsets / masked_m (ignored for weights);
    bad_count: optional int32 [1] device tensor the kernel adds the number of
    active non-UE8M0 scales to.  Returns the packed uint8 tensor."""
    torch = _torch()
    dev = scales.device
    if scales.dtype not in (torch.float32, torch.uint8):
        raise TypeError("scales must be float32 or uint8 (E8M0 bytes)")
    if not scales.is_contiguous():
        raise ValueError("scales must be contiguous")
    if groups is not None:
        _check(groups, "groups", torch.int32, 1, dev)
    nbytes = fp8_scale_bytes(layout, rows, k, num_groups)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(out, "out", torch.uint8, 1, dev)
    if out.numel() < nbytes:
        raise ValueError(f"out must hold {nbytes} bytes")
    if bad_count is not None:
        _check(bad_count, "bad_count", torch.int32, 1, dev)
    rc = call_raw("gg_fp8_pack_scales", int(layout), scales.data_ptr(),
                  1 if scales.dtype == torch.float32 else 0, int(scales.shape[-1]),
                  None if groups is None else groups.data_ptr(), int(rows), int(k), int(num_groups),
                  out.data_ptr(), None if bad_count is None else bad_count.data_ptr(),
                  _stream_handle(dev))
    if rc != 0:
        raise GGError("gg_fp8_pack_scales", rc, last_error())
    return out


def _fp8_call(name, x, xs, w, ws, groups, out, m, k, n, e, dev):
    rc = call_raw(name, x.data_ptr(), xs.data_ptr(), w.data_ptr(), ws.data_ptr(), groups.data_ptr(),
                  out.data_ptr(), _dtype_code(out.dtype), int(m), int(k), int(n), int(e),
                  _stream_handle(dev))
    if rc != 0:
        raise GGError(name, rc, last_error())


def fp8_forward(x, x_scales, w, w_scales, offs, out=None, out_dtype=None):
    """Y[rows of g] = sum_k x sx w[g] sw over 128-value scale blocks
    (gg_fp8_forward).  x: uint8 e4m3 [m, k]; w: uint8 e4m3 [E, n, k];
    x_scales / w_scales: packed by fp8_pack_scales (GG_FP8_ACT_RAGGED with
    the same offs / GG_FP8_WEIGHT); offs: int32 [E] end offsets."""
    torch = _torch()
    dev = x.device
    _check(x, "x", torch.uint8, 2, dev)
    _check(w, "w", torch.uint8, 3, dev)
    _check(offs, "offs", torch.int32, 1, dev)
    _check(x_scales, "x_scales", torch.uint8, 1, dev)
    _check(w_scales, "w_scales", torch.uint8, 1, dev)
    m, k = x.shape
    e, n, k2 = w.shape
    if k2 != k or offs.shape[0] != e:
        raise ValueError("shape mismatch between x, w and offs")
    if x_scales.numel() < fp8_scale_bytes(GG_FP8_ACT_RAGGED, m, k, e) or \
            w_scales.numel() < fp8_scale_bytes(GG_FP8_WEIGHT, n, k, e):
        raise ValueError("packed scales are smaller than fp8_scale_bytes requires")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype or torch.bfloat16, device=dev)
    _check(out, "out", out.dtype, 2, dev)
    if tuple(out.shape) != (m, n):
        raise ValueError(f"out must be [{m}, {n}]")
    _fp8_call("gg_fp8_forward", x, x_scales, w, w_scales, offs, out, m, k, n, e, dev)
    return out


def fp8_masked_forward(x, x_scales, w, w_scales, masked_m, out=None, out_dtype=None):
    """The masked fp8 forward (gg_fp8_masked_forward): x uint8 [E, max_m, k],
    x_scales packed with GG_FP8_ACT_MASKED and the same masked_m."""
    torch = _torch()
    dev = x.device
    _check(x, "x", torch.uint8, 3, dev)
    _check(w, "w", torch.uint8, 3, dev)
    _check(masked_m, "masked_m", torch.int32, 1, dev)
    _check(x_scales, "x_scales", torch.uint8, 1, dev)
    _check(w_scales, "w_scales", torch.uint8, 1, dev)
    e, max_m, k = x.shape
    e2, n, k2 = w.shape
    if e2 != e or k2 != k or masked_m.shape[0] != e:
        raise ValueError("shape mismatch between x, w and masked_m")
    if x_scales.numel() < fp8_scale_bytes(GG_FP8_ACT_MASKED, max_m, k, e) or \
            w_scales.numel() < fp8_scale_bytes(GG_FP8_WEIGHT, n, k, e):
        raise ValueError("packed scales are smaller than fp8_scale_bytes requires")
    if out is None:
        out = torch.empty((e, max_m, n), dtype=out_dtype or torch.bfloat16, device=dev)
    _check(out, "out", out.dtype, 3, dev)
    if tuple(out.shape) != (e, max_m, n):
        raise ValueError(f"out must be [{e}, {max_m}, {n}]")
    _fp8_call("gg_fp8_masked_forward", x, x_scales, w, w_scales, masked_m, out, max_m, k, n, e, dev)
    return out
