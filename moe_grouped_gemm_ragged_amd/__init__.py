"""bf16 grouped (ragged, per-expert) GEMM for MoE layers on MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
include/gg.h (libgg.so, built in-tree by ``moe_grouped_gemm_ragged_amd.build``).
This package holds the thin ctypes binding (``binding``) and the seeded
synthetic workloads (``synth``).
"""
from .binding import (GG_BF16, GG_F32, GGError, dgrad, forward, load, masked_forward,
                      wgrad)

__all__ = ["forward", "dgrad", "wgrad", "masked_forward", "load", "GGError",
           "GG_BF16", "GG_F32"]
__version__ = "0.1.0"
