"""wgrad reads X and dY down each expert's rows, one 32-bit buffer range per
stage running to the expert's last row; an expert can span 4 GB or more of
either, and the range must not wrap:

* one ragged expert of 270000 rows at k = 8192 (X spans 4.4 GB) after a
  short one (fp32 and bf16 dW), the same rows as one masked expert, and 32
  short experts at k = 65536 (the staged fp32 epilogue);
* at the boundary of the weight limit (k * n just under 2^31), the forward,
  which reads W[g] down its k rows through ranges just under 4 GB.

The inputs are small periodic integers (period 3 along one index, 5 along
the other, values in {-2 .. 2}), so every output is an exact integer below
2^24 that a residue count gives in closed form: a reduction row dropped,
repeated or taken from the wrong place anywhere changes the bits.
"""
import numpy as np
import pytest

from moe_grouped_gemm_ragged_amd import binding as gg
from gpu_util import device, say

pytestmark = pytest.mark.gpu

X3 = np.array([-1, 0, 1], dtype=np.int64)          # x = X3[(i + j) mod 3]
D5 = np.array([-2, -1, 0, 1, 2], dtype=np.int64)   # d = D5[(7 i + j) mod 5]


def _periodic(rows, cols, table, mult, dev):
    """[rows, cols] bf16 with element (i, j) = table[(mult * i + j) mod p]."""
    import torch
    p = len(table)
    pat = np.array([[table[(mult * c + j) % p] for j in range(cols)] for c in range(p)], dtype=np.float32)
    idx = torch.arange(rows, device=dev) % p
    return torch.from_numpy(pat).to(dev).to(torch.bfloat16).index_select(0, idx)


def _residue_counts(lo, hi, period=15):
    """How many i in [lo, hi) have i mod period == c, for each c."""
    c = np.arange(period)
    return (hi - c + period - 1) // period - (lo - c + period - 1) // period


# (layout, expert sizes, rows m, k, output dtype).  The last case has short
# experts (1024 rows: the LDS-staged fp32 epilogue) while m * 2k still
# passes 2^32, so the capped ranges run there too.
WGRAD_CASES = {
    "ragged_f32": ("ragged", [8, 270000], 270008, 8192, "f32"),
    "ragged_bf16": ("ragged", [8, 270000], 270008, 8192, "bf16"),
    "masked_f32": ("masked", [269993], 270000, 8192, "f32"),
    "short_experts_f32": ("ragged", [1024] * 32, 32768, 65536, "f32"),
}


@pytest.mark.parametrize("case", list(WGRAD_CASES))
def test_wgrad_expert_span_over_4gb(case):
    import torch
    dev = device()
    layout, sizes, m, k, out = WGRAD_CASES[case]
    n = 64
    assert m * 2 * k >= 2 ** 32
    say("wgrad large span", case, m, k, n)
    x = _periodic(m, k, X3, 1, dev)          # x[r, kk] = X3[(r + kk) mod 3]
    dy = _periodic(m, n, D5, 7, dev)         # dy[r, j] = D5[(7 r + j) mod 5]
    odt = torch.float32 if out == "f32" else torch.bfloat16
    if layout == "ragged":
        ends = np.cumsum(sizes)
        ranges = list(zip([0] + ends[:-1].tolist(), ends.tolist()))
        offs = torch.from_numpy(ends.astype(np.int32)).to(dev)
        dw = gg.wgrad(x, dy, offs, out_dtype=odt)
    else:
        ranges = [(0, sizes[0])]
        mm = torch.tensor(sizes, dtype=torch.int32, device=dev)
        dw = gg.masked_wgrad(x.view(1, m, k), dy.view(1, m, n), mm, out_dtype=odt)
    torch.cuda.synchronize()
    # every expert, on a fixed sample of 1024 k rows (all k rows when k <= 8192)
    ks = np.arange(k) if k <= 8192 else np.sort(np.random.default_rng(5).choice(k, 1024, replace=False))
    sel = dw[:, torch.from_numpy(ks).to(dev)]
    got = (sel.view(torch.int16) if odt == torch.bfloat16 else sel).cpu().numpy()
    del x, dy, dw, sel
    torch.cuda.empty_cache()
    kk = ks[:, None]
    jj = np.arange(n)[None, :]
    for g, (lo, hi) in enumerate(ranges):
        cnt = _residue_counts(lo, hi)
        want = np.zeros((len(ks), n), dtype=np.int64)
        for c in range(15):
            want += cnt[c] * X3[(c + kk) % 3] * D5[(7 * c + jj) % 5]
        assert np.abs(want).max() < 2 ** 24
        w32 = want.astype(np.float32)
        if odt == torch.bfloat16:
            # exact fp32 sums, one rounding to bf16 (round to nearest even)
            w32 = torch.from_numpy(w32).to(torch.bfloat16).view(torch.int16).numpy()
        bad = np.argwhere(got[g] != w32)
        assert bad.size == 0, f"expert {g}: {len(bad)} wrong dW entries, first {bad[:3].tolist()}"


def test_forward_weight_at_the_size_limit():
    import torch
    dev = device()
    k, n, m = 65536, 32760, 300
    assert k * n < 2 ** 31 and (k - 1) * 2 * n + 2 * n > 2 ** 32 - 2 ** 21
    say("forward weight at the limit", m, k, n)
    x = _periodic(m, k, X3, 1, dev)          # x[r, kk] = X3[(r + kk) mod 3]
    w = _periodic(k, n, D5, 7, dev)          # w[kk, j] = D5[(7 kk + j) mod 5]
    offs = torch.tensor([m], dtype=torch.int32, device=dev)
    y = gg.forward(x, w.view(1, k, n), offs)
    torch.cuda.synchronize()
    got = y.view(torch.int16).cpu().numpy()
    del x, w, y
    torch.cuda.empty_cache()
    cnt = _residue_counts(0, k)
    rr = np.arange(m)[:, None]
    jj = np.arange(n)[None, :]
    want = np.zeros((m, n), dtype=np.int64)
    for c in range(15):
        want += cnt[c] * X3[(rr + c) % 3] * D5[(7 * c + jj) % 5]
    assert np.abs(want).max() < 2 ** 24
    # exact fp32 sums, one rounding to bf16 (round to nearest even)
    want_bits = torch.from_numpy(want.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    bad = np.argwhere(got != want_bits)
    assert bad.size == 0, f"{len(bad)} wrong Y entries, first {bad[:3].tolist()}"
