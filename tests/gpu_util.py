"""Helpers shared by the GPU tests (test infrastructure)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from moe_grouped_gemm_ragged_amd import synth

SENT_BF16 = synth.OUT_SENTINEL_BF16
SENT_F32 = synth.OUT_SENTINEL_F32


def device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def say(*args):
    """Name the case before each GPU step, flushed, so a crash still shows it."""
    print("[gpu-test]", *args, file=sys.stderr, flush=True)


def sentinel_tensor(shape, dtype, dev):
    import torch
    if dtype == torch.bfloat16:
        v = int(np.array([SENT_BF16], dtype=np.uint16).view(np.int16)[0])
        return torch.full(shape, v, dtype=torch.int16, device=dev).view(torch.bfloat16)
    v = int(np.array([SENT_F32], dtype=np.uint32).view(np.int32)[0])
    return torch.full(shape, v, dtype=torch.int32, device=dev).view(torch.float32)


def nan_tensor(shape, dtype, dev):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype, device=dev)


def host(t) -> np.ndarray:
    """bf16 -> uint16 bit patterns, fp32 -> float32, on the host."""
    import torch
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits(t)
    return t.detach().contiguous().cpu().numpy()


def sentinel_bits(dtype):
    import torch
    return SENT_BF16 if dtype == torch.bfloat16 else SENT_F32


def raw_bits(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return a
    return a.view(np.uint32)
