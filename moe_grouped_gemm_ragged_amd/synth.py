"""Seeded synthetic workloads for the bf16 grouped (ragged, per-expert) GEMM.

This module holds shapes, group-size recipes and random draws only: none of
the GEMM's arithmetic lives here, so the CPU oracle and the HIP path can both
take their inputs from it without sharing any of the method.

Shapes and group-size structure follow the workloads the pages describe:

* ``tiny``: the minimal reproduction of the empty-expert backward hang in
  PyTorch issue #152668 (section "Easy repro scenario"): 4 experts,
  X [48, 8], W [4, 8, 16], end offsets (8, 8, 32, 40), so expert 1 is empty
  and rows 40..47 are unused.
* ``qwen3_gateup``: Qwen3-30B-A3B gate/up projection (sglang PR #32385,
  section "Cause", model table: moe_intermediate 768, i.e. N = 2*768): 128
  experts, K = 2048, N = 1536, 8192 tokens x top-8 = 65536 rows.
* ``masked_down``: the masked down-projection of sglang PR #32385 (section
  "Evidence", operand table: 64 experts x 256 rows, K = 768, N = 2048).
* ``glm_up``: the GLM-up shape of TileOPs issue #1566 (section "Summary":
  numel = 262144, N = 4096, K = 6144), 32 experts with 128-aligned sizes.
* ``dsv3``: a DeepSeek-V3-class layer (sglang PR #32385, model table:
  moe_intermediate 2048): 256 experts, K = 7168, N = 2048, 32768 rows with
  Zipf-skewed sizes and about 10 % empty experts.

The ``*_small`` variants keep each recipe's structure (empty groups, sizes 8
and 16, unaligned tails, NaN in inactive rows) at sizes a plain CPU loop
finishes in seconds while still spanning several 256 x 256 tiles.

Tensors are drawn with ``torch.randn`` from a ``torch.Generator`` seeded per
tensor, on the device the caller names, then rounded to bf16 by torch's
round-to-nearest-even cast.  Group sizes are drawn on the host with numpy and
are identical on every device.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

# bf16 bit patterns used as markers in never-read / never-written regions.
BF16_QNAN = 0x7FC0
OUT_SENTINEL_BF16 = 0xDEAD          # a finite bf16 (about -6.2e18)
OUT_SENTINEL_F32 = 0xDEADBEEF       # a finite fp32 (about -6.3e18)


@dataclass
class Workload:
    """One grouped-GEMM problem: shapes, group structure and draw recipe."""

    name: str
    layout: str                      # "ragged" (end offsets) or "masked"
    num_groups: int
    m: int                           # ragged: rows of X; masked: max_m
    k: int
    n: int
    seed: int
    offs: Optional[np.ndarray] = None        # int32 [E], ragged only
    masked_m: Optional[np.ndarray] = None    # int32 [E], masked only
    x_std: float = 1.0
    w_std: float = 0.02
    dy_std: float = 1.0
    notes: Dict[str, str] = field(default_factory=dict)

    # --- derived sizes -------------------------------------------------
    def group_sizes(self) -> np.ndarray:
        if self.layout == "masked":
            return np.minimum(np.maximum(self.masked_m.astype(np.int64), 0), self.m)
        ends = self.offs.astype(np.int64)
        starts = np.concatenate([[0], ends[:-1]])
        return ends - starts

    def active_rows(self) -> int:
        return int(self.group_sizes().sum())

    def flops(self) -> int:
        """2 * (active rows) * K * N: the FLOP count of one pass."""
        return 2 * self.active_rows() * self.k * self.n

    def x_shape(self):
        if self.layout == "masked":
            return (self.num_groups, self.m, self.k)
        return (self.m, self.k)

    def w_shape(self):
        return (self.num_groups, self.k, self.n)

    def y_shape(self):
        if self.layout == "masked":
            return (self.num_groups, self.m, self.n)
        return (self.m, self.n)


# ---------------------------------------------------------------------------
# group-size recipes (host, numpy)
# ---------------------------------------------------------------------------

def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream]))


def _ends(sizes) -> np.ndarray:
    return np.cumsum(np.asarray(sizes, dtype=np.int64)).astype(np.int32)


def _force_sizes(sizes: np.ndarray, forced: Dict[int, int]) -> np.ndarray:
    """Set sizes[i] = v for each forced entry and move the difference onto
    the largest unforced group, so the total is unchanged."""
    sizes = sizes.astype(np.int64).copy()
    total = int(sizes.sum())
    for i, v in forced.items():
        sizes[i] = v
    free = [i for i in range(len(sizes)) if i not in forced]
    big = max(free, key=lambda i: sizes[i])
    sizes[big] += total - int(sizes.sum())
    assert sizes[big] >= 0 and int(sizes.sum()) == total
    return sizes


def softmax_multinomial_sizes(num_groups: int, rows: int, seed: int,
                              n_zero: int = 3, n_eight: int = 1,
                              n_sixteen: int = 1) -> np.ndarray:
    """Routing-like sizes: Multinomial(rows, softmax(N(0,1) logits)), then a
    few experts forced to 0, 8 and 16 rows (the sizes that hung the
    backward in PyTorch issue #152668, section "Describe the bug")."""
    r = _rng(seed, 1)
    logits = r.standard_normal(num_groups)
    p = np.exp(logits - logits.max())
    p /= p.sum()
    sizes = r.multinomial(rows, p)
    pick = r.permutation(num_groups)
    forced = {}
    j = 0
    for count, val in ((n_zero, 0), (n_eight, 8), (n_sixteen, 16)):
        for _ in range(count):
            forced[int(pick[j])] = val
            j += 1
    return _force_sizes(sizes, forced)


def dirichlet_aligned_sizes(num_groups: int, rows: int, align: int,
                            seed: int) -> np.ndarray:
    """Dirichlet(1) proportions, rounded to multiples of ``align`` by the
    largest-remainder rule so the sizes sum exactly to ``rows``."""
    assert rows % align == 0
    units_total = rows // align
    r = _rng(seed, 2)
    p = r.dirichlet(np.ones(num_groups))
    raw = p * units_total
    units = np.floor(raw).astype(np.int64)
    rem = units_total - int(units.sum())
    order = np.argsort(-(raw - units), kind="stable")
    units[order[:rem]] += 1
    assert int(units.sum()) == units_total
    return units * align


def zipf_sizes(num_groups: int, rows: int, seed: int, s: float = 1.1,
               empty_frac: float = 0.10) -> np.ndarray:
    """Zipf(s)-skewed sizes over a random rank order, with ``empty_frac`` of
    the experts forced empty (they get probability zero)."""
    r = _rng(seed, 3)
    n_empty = int(round(empty_frac * num_groups))
    perm = r.permutation(num_groups)
    empty = perm[:n_empty]
    live = perm[n_empty:]
    ranks = np.arange(1, len(live) + 1, dtype=np.float64)
    w = ranks ** (-s)
    p = np.zeros(num_groups)
    p[live] = w / w.sum()
    sizes = r.multinomial(rows, p)
    sizes[empty] = 0
    return sizes.astype(np.int64)


def uniform_masked_m(num_groups: int, max_m: int, seed: int,
                     n_zero: int = 2, n_eight: int = 2,
                     n_full: int = 1) -> np.ndarray:
    """masked_m ~ U{0..max_m}, with some experts forced to 0, 8 and max_m."""
    r = _rng(seed, 4)
    mm = r.integers(0, max_m + 1, size=num_groups)
    pick = r.permutation(num_groups)
    j = 0
    for count, val in ((n_zero, 0), (n_eight, 8), (n_full, max_m)):
        for _ in range(count):
            if j < num_groups:
                mm[pick[j]] = val
                j += 1
    return mm.astype(np.int32)


# ---------------------------------------------------------------------------
# the workloads
# ---------------------------------------------------------------------------

def tiny() -> Workload:
    return Workload("tiny", "ragged", 4, 48, 8, 16, seed=1,
                    offs=np.array([8, 8, 32, 40], dtype=np.int32),
                    x_std=1.0, w_std=1.0, dy_std=1.0,
                    notes={"source": "PyTorch issue #152668, Easy repro scenario"})


def qwen3_gateup(scale: str = "full") -> Workload:
    if scale == "full":
        E, M, K, N, seed = 128, 65536, 2048, 1536, 2
    else:
        E, M, K, N, seed = 16, 4096, 512, 384, 12
    sizes = softmax_multinomial_sizes(E, M, seed)
    return Workload("qwen3_gateup" + ("" if scale == "full" else "_small"),
                    "ragged", E, M, K, N, seed=seed, offs=_ends(sizes))


def masked_down(scale: str = "full") -> Workload:
    if scale == "full":
        E, MAXM, K, N, seed = 64, 256, 768, 2048, 3
    else:
        E, MAXM, K, N, seed = 8, 256, 256, 320, 13
    mm = uniform_masked_m(E, MAXM, seed)
    return Workload("masked_down" + ("" if scale == "full" else "_small"),
                    "masked", E, MAXM, K, N, seed=seed, masked_m=mm)


def glm_up(scale: str = "full") -> Workload:
    if scale == "full":
        E, M, K, N, seed = 32, 262144, 6144, 4096, 4
    else:
        E, M, K, N, seed = 8, 4096, 384, 512, 14
    sizes = dirichlet_aligned_sizes(E, M, 128, seed)
    return Workload("glm_up" + ("" if scale == "full" else "_small"),
                    "ragged", E, M, K, N, seed=seed, offs=_ends(sizes))


def dsv3(scale: str = "full") -> Workload:
    if scale == "full":
        E, M, K, N, seed = 256, 32768, 7168, 2048, 5
    else:
        E, M, K, N, seed = 32, 2048, 456, 328, 15
    sizes = zipf_sizes(E, M, seed)
    return Workload("dsv3" + ("" if scale == "full" else "_small"),
                    "ragged", E, M, K, N, seed=seed, offs=_ends(sizes))


FULL = {"tiny": tiny, "qwen3_gateup": qwen3_gateup, "masked_down": masked_down,
        "glm_up": glm_up, "dsv3": dsv3}


def by_name(name: str) -> Workload:
    if name.endswith("_small"):
        return FULL[name[: -len("_small")]]("small")
    return FULL[name]()


def custom_ragged(name: str, sizes, k: int, n: int, seed: int, m: Optional[int] = None,
                  x_std=1.0, w_std=0.02, dy_std=1.0) -> Workload:
    """A ragged workload with explicit group sizes; ``m`` may exceed the sum
    (unused trailing rows)."""
    ends = _ends(sizes)
    m = int(ends[-1]) if m is None else m
    return Workload(name, "ragged", len(ends), m, k, n, seed=seed, offs=ends,
                    x_std=x_std, w_std=w_std, dy_std=dy_std)


def custom_masked(name: str, masked_m, max_m: int, k: int, n: int, seed: int,
                  x_std=1.0, w_std=0.02) -> Workload:
    mm = np.asarray(masked_m, dtype=np.int32)
    return Workload(name, "masked", len(mm), max_m, k, n, seed=seed, masked_m=mm,
                    x_std=x_std, w_std=w_std)


# ---------------------------------------------------------------------------
# tensor draws (torch; device chosen by the caller)
# ---------------------------------------------------------------------------

def _randn_bf16(shape, std: float, seed: int, stream: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + stream)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def make_inputs(wl: Workload, device="cpu", need=("x", "w", "dy")):
    """Draw the bf16 operands of ``wl`` on ``device``.

    Returns a dict with any of ``x``, ``w``, ``dy`` (bf16 tensors) and
    ``offs`` / ``masked_m`` (int32 tensors).  For the masked layout the
    inactive rows of X and dY hold bf16 quiet NaN, so a read of them would
    show.
    """
    import torch
    out = {}
    if "x" in need:
        x = _randn_bf16(wl.x_shape(), wl.x_std, wl.seed, 1, device)
        if wl.layout == "masked":
            sizes = wl.group_sizes()
            xi = x.view(torch.int16)
            for e in range(wl.num_groups):
                xi[e, int(sizes[e]):, :] = BF16_QNAN
        out["x"] = x
    if "w" in need:
        out["w"] = _randn_bf16(wl.w_shape(), wl.w_std, wl.seed, 2, device)
    if "dy" in need:
        if wl.layout == "masked":
            dy = _randn_bf16((wl.num_groups, wl.m, wl.n), wl.dy_std, wl.seed, 3, device)
            sizes = wl.group_sizes()
            dyi = dy.view(torch.int16)
            for e in range(wl.num_groups):
                dyi[e, int(sizes[e]):, :] = BF16_QNAN
            out["dy"] = dy
        else:
            out["dy"] = _randn_bf16((wl.m, wl.n), wl.dy_std, wl.seed, 3, device)
    if wl.layout == "masked":
        out["masked_m"] = torch.from_numpy(wl.masked_m.astype(np.int32)).to(device)
    else:
        out["offs"] = torch.from_numpy(wl.offs.astype(np.int32)).to(device)
    return out


# ---------------------------------------------------------------------------
# fp8 (e4m3) operands with power-of-two block scales
# ---------------------------------------------------------------------------

E4M3_NAN = 0x7F                     # the e4m3 NaN code, marker for never-read rows
SCALE_GARBAGE_F32 = 0.3             # a non-power-of-two scale, marker for never-read rows


def fp8_masked_down(scale: str = "full") -> Workload:
    """The masked down-projection of sglang PR #32385 in fp8 (its fp8
    rollout: "Evidence", operand table, down A/B: 64 experts x 256 rows,
    K = 768 (G = 6 scale blocks), N = 2048)."""
    if scale == "full":
        E, MAXM, K, N, seed = 64, 256, 768, 2048, 21
    else:
        E, MAXM, K, N, seed = 8, 256, 256, 320, 31
    mm = uniform_masked_m(E, MAXM, seed)
    return Workload("fp8_masked_down" + ("" if scale == "full" else "_small"),
                    "masked", E, MAXM, K, N, seed=seed, masked_m=mm)


def fp8_masked_gateup(scale: str = "full") -> Workload:
    """The masked gate/up projection of the same step (operand table,
    gateup A/B: 64 experts x 256 rows, K = 2048 (G = 16), N = 1536)."""
    if scale == "full":
        E, MAXM, K, N, seed = 64, 256, 2048, 1536, 22
    else:
        E, MAXM, K, N, seed = 8, 256, 384, 384, 32
    mm = uniform_masked_m(E, MAXM, seed)
    return Workload("fp8_masked_gateup" + ("" if scale == "full" else "_small"),
                    "masked", E, MAXM, K, N, seed=seed, masked_m=mm)


def fp8_repro() -> Workload:
    """The minimal reproduction of sglang PR #32385 ("Evidence" 1): 8
    experts, max_m 128, K = 768, N = 2048, 8 active rows per expert."""
    return Workload("fp8_repro", "masked", 8, 128, 768, 2048, seed=23,
                    masked_m=np.full(8, 8, dtype=np.int32))


def fp8_qwen3_gateup(scale: str = "full") -> Workload:
    """The ragged Qwen3 gate/up recipe (see qwen3_gateup) in fp8."""
    wl = qwen3_gateup(scale)
    wl.name = "fp8_" + wl.name
    return wl


def fp8_glm_up(scale: str = "full") -> Workload:
    """The GLM-up recipe (see glm_up) in fp8."""
    wl = glm_up(scale)
    wl.name = "fp8_" + wl.name
    return wl


FULL.update({"fp8_masked_down": fp8_masked_down, "fp8_masked_gateup": fp8_masked_gateup,
             "fp8_repro": lambda scale="full": fp8_repro(),
             "fp8_qwen3_gateup": fp8_qwen3_gateup, "fp8_glm_up": fp8_glm_up})


def _quantize_e4m3_blocks(t):
    """Per row and per 128 values along the last dim: a power-of-two scale
    2^ceil(log2(amax / 448)) (1.0 for an all-zero block; the rounding rule of
    the quantizer in sglang PR #32385, "Cause") and the e4m3 codes of t /
    scale by torch's cast.  Returns (uint8 codes, fp32 scales [..., G])."""
    import torch
    *lead, k = t.shape
    g = (k + 127) // 128
    pad = g * 128 - k
    tp = torch.nn.functional.pad(t, (0, pad)) if pad else t
    blocks = tp.reshape(*lead, g, 128)
    amax = blocks.abs().amax(dim=-1)
    scale = torch.where(amax > 0, torch.exp2(torch.ceil(torch.log2(amax / 448.0))),
                        torch.ones_like(amax))
    q = (blocks / scale.unsqueeze(-1)).reshape(*lead, g * 128)[..., :k]
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.to(torch.float32).contiguous()


def make_fp8_inputs(wl: Workload, device="cpu"):
    """Draw the fp8 operands of ``wl`` on ``device``: ``x8`` uint8 e4m3
    [M, K] (masked: [E, max_m, K]) with ``sx`` fp32 [..., ceil(K/128)], and
    ``w8`` uint8 e4m3 [E, N, K] (K contiguous) with ``sw`` fp32
    [E, N, ceil(K/128)]; every scale a power of two.  In the masked layout
    the inactive rows hold the e4m3 NaN code and the non-power-of-two scale
    0.3, so a read of either would show."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(wl.seed) * 1000003 + 11)
    x = torch.randn(wl.x_shape(), generator=g, device=device, dtype=torch.float32) * wl.x_std
    g.manual_seed(int(wl.seed) * 1000003 + 12)
    w = torch.randn((wl.num_groups, wl.n, wl.k), generator=g, device=device,
                    dtype=torch.float32) * wl.w_std
    x8, sx = _quantize_e4m3_blocks(x)
    del x
    w8, sw = _quantize_e4m3_blocks(w)
    del w
    out = {"x8": x8, "sx": sx, "w8": w8, "sw": sw}
    if wl.layout == "masked":
        sizes = wl.group_sizes()
        for e in range(wl.num_groups):
            x8[e, int(sizes[e]):, :] = E4M3_NAN
            sx[e, int(sizes[e]):, :] = SCALE_GARBAGE_F32
        out["masked_m"] = torch.from_numpy(wl.masked_m.astype(np.int32)).to(device)
    else:
        out["offs"] = torch.from_numpy(wl.offs.astype(np.int32)).to(device)
    return out


def bf16_bits(t) -> np.ndarray:
    """A bf16 torch tensor's bit patterns as a host uint16 array."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
