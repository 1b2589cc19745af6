"""GPU parity of the fp8 (e4m3) block-scaled forward against the fp64 oracle.

* scale packing (gg_fp8_pack_scales) + forward on scaled-down ragged and
  masked workloads, every row, bf16 and fp32 outputs, sentinel-filled
  outputs (rows outside the experts, or inactive, come back untouched);
* inactive rows holding the e4m3 NaN code and non-power-of-two scales are
  never read: the output equals that of zeros there, and the validity count
  ignores them;
* the validity count over active rows equals the oracle's count;
* E8M0 byte scales (the packed int32 form, G padded to a multiple of 4)
  give bit-identical results to the same scales as fp32;
* edge cases: empty experts, one-row experts, a ragged row tail, k = 128
  (one scale block), a column tail, half-height last tiles;
* the full-size Qwen3 gate/up shape and the masked down and gate/up
  projections of the page's operand table, every element, and the GLM-up
  shape on sampled rows (every expert's first and last rows and its tile
  boundaries, plus random rows), in the benchmark's launch configuration.
Tolerance: parity.check_fp8.
"""
import numpy as np
import pytest

import oracle
from moe_grouped_gemm_ragged_amd import binding as gg
from moe_grouped_gemm_ragged_amd import synth
from gpu_util import device, host, raw_bits, say, sentinel_bits, sentinel_tensor
from parity import Report, check_fp8

pytestmark = pytest.mark.gpu


def _dt(name):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def run_fp8(wl, t, out):
    """Pack both operands' scales and run the fp8 forward into `out`."""
    e = wl.num_groups
    ws = gg.fp8_pack_scales(gg.GG_FP8_WEIGHT, t["sw"], None, wl.n, wl.k, e)
    if wl.layout == "masked":
        xs = gg.fp8_pack_scales(gg.GG_FP8_ACT_MASKED, t["sx"], t["masked_m"], wl.m, wl.k, e)
        gg.fp8_masked_forward(t["x8"], xs, t["w8"], ws, t["masked_m"], out=out)
    else:
        xs = gg.fp8_pack_scales(gg.GG_FP8_ACT_RAGGED, t["sx"], t["offs"], wl.m, wl.k, e)
        gg.fp8_forward(t["x8"], xs, t["w8"], ws, t["offs"], out=out)
    return out


def oracle_fp8(wl, t, rows=None):
    x8, sx = t["x8"].cpu().numpy(), t["sx"].cpu().numpy()
    w8, sw = t["w8"].cpu().numpy(), t["sw"].cpu().numpy()
    if wl.layout == "masked":
        return oracle.fp8_masked_forward(x8, sx, w8, sw, wl.masked_m, rows=rows)
    return oracle.fp8_forward(x8, sx, w8, sw, wl.offs, rows=rows)


def out_shape(wl):
    return (wl.num_groups, wl.m, wl.n) if wl.layout == "masked" else (wl.m, wl.n)


def check_all_rows(wl, t, y, what):
    import torch
    torch.cuda.synchronize()
    ref = oracle_fp8(wl, t)
    yh = host(y).reshape(-1, wl.n)
    used = ref.status == 1
    rep = Report()
    check_fp8(yh[used], ref.value[used], ref.sabs[used], wl.k, what, rep)
    assert np.all(raw_bits(yh[~used]) == sentinel_bits(y.dtype)), f"{what}: rows outside the experts were written"
    print(what, rep)


SMALL = ["fp8_masked_down_small", "fp8_masked_gateup_small", "fp8_qwen3_gateup_small",
         "fp8_glm_up_small", "fp8_repro"]


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("name", SMALL)
def test_fp8_forward_small(name, out):
    dev = device()
    wl = synth.by_name(name)
    t = synth.make_fp8_inputs(wl, dev)
    y = sentinel_tensor(out_shape(wl), _dt(out), dev)
    say("fp8 forward", name, out)
    run_fp8(wl, t, y)
    check_all_rows(wl, t, y, f"fp8 {name} {out}")


@pytest.mark.parametrize("sizes,k,n,tail", [
    ([0, 1, 128, 129, 0, 300, 7], 128, 264, 5),
    ([256, 0, 0, 513, 64], 384, 200, 0),
    ([1] * 12, 256, 64, 3),
])
def test_fp8_forward_ragged_edges(sizes, k, n, tail):
    dev = device()
    wl = synth.custom_ragged("fp8_edges", sizes, k, n, seed=41 + k, m=int(sum(sizes)) + tail)
    t = synth.make_fp8_inputs(wl, dev)
    y = sentinel_tensor((wl.m, wl.n), _dt("bf16"), dev)
    say("fp8 ragged edges", sizes, k, n, tail)
    run_fp8(wl, t, y)
    check_all_rows(wl, t, y, f"fp8 edges {sizes} k={k} n={n}")


def test_fp8_masked_inactive_rows_never_read():
    dev = device()
    import torch
    wl = synth.by_name("fp8_masked_down_small")
    t = synth.make_fp8_inputs(wl, dev)          # inactive rows: NaN codes, scale 0.3
    clean = {k: v.clone() for k, v in t.items()}
    sizes = wl.group_sizes()
    for e in range(wl.num_groups):
        clean["x8"][e, int(sizes[e]):] = 0
        clean["sx"][e, int(sizes[e]):] = 1.0
    say("fp8 masked inactive rows")
    bad = torch.zeros(1, dtype=torch.int32, device=dev)
    xs = gg.fp8_pack_scales(gg.GG_FP8_ACT_MASKED, t["sx"], t["masked_m"], wl.m, wl.k, wl.num_groups,
                            bad_count=bad)
    ws = gg.fp8_pack_scales(gg.GG_FP8_WEIGHT, t["sw"], None, wl.n, wl.k, wl.num_groups, bad_count=bad)
    y1 = sentinel_tensor(out_shape(wl), torch.bfloat16, dev)
    gg.fp8_masked_forward(t["x8"], xs, t["w8"], ws, t["masked_m"], out=y1)
    y2 = sentinel_tensor(out_shape(wl), torch.bfloat16, dev)
    run_fp8(wl, clean, y2)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0, "inactive scales were validated"
    assert np.array_equal(host(y1), host(y2)), "inactive rows changed the result"
    check_all_rows(wl, t, y1, "fp8 masked with garbage in inactive rows")


@pytest.mark.parametrize("case", ["masked_scalar", "masked_vec", "ragged_vec"])
def test_fp8_bad_scale_count_matches_oracle(case):
    """Three non-UE8M0 scales planted in active rows are counted, and the
    garbage in inactive rows (masked: past masked_m; ragged: capacity rows
    past the last offset) is not.  K = 384 reads one scale per load; K = 1024
    (8 k-blocks) takes the four-scales-per-load path."""
    dev = device()
    import torch
    if case == "masked_scalar":
        wl = synth.by_name("fp8_masked_gateup_small")
    elif case == "masked_vec":
        wl = synth.custom_masked("fp8_bad_vec", synth.uniform_masked_m(8, 256, 43), 256, 1024, 256, seed=43)
    else:
        sizes = np.array([300, 0, 77, 512, 129], dtype=np.int64)
        wl = synth.custom_ragged("fp8_bad_ragged", sizes, 1024, 256, seed=44, m=int(sizes.sum()) + 40)
    t = synth.make_fp8_inputs(wl, dev)
    sizes = wl.group_sizes()
    sx = t["sx"]
    if wl.layout == "masked":
        live = [e for e in range(wl.num_groups) if sizes[e] > 2]
        sx[live[0], 0, 0] = 0.3
        sx[live[1], 1, 1] = -1.0
        sx[live[-1], int(sizes[live[-1]]) - 1, 2] = 1.5
        active = np.arange(wl.m)[None, :, None] < sizes[:, None, None]
        layout, groups = gg.GG_FP8_ACT_MASKED, t["masked_m"]
    else:
        end = int(sizes.sum())
        sx[end:, :] = 0.3                      # capacity rows: never validated
        sx[0, 0] = 0.3
        sx[350, 5] = -1.0
        sx[end - 1, 7] = 1.5
        active = (np.arange(wl.m) < end)[:, None]
        layout, groups = gg.GG_FP8_ACT_RAGGED, t["offs"]
    want = oracle.ue8m0_violations(sx.cpu().numpy(), np.broadcast_to(active, sx.shape))
    say("fp8 bad scale count", case)
    bad = torch.zeros(1, dtype=torch.int32, device=dev)
    gg.fp8_pack_scales(layout, sx, groups, wl.m, wl.k, wl.num_groups, bad_count=bad)
    torch.cuda.synchronize()
    assert want == 3
    assert int(bad.item()) == want


def test_fp8_e8m0_byte_scales_match_fp32_scales():
    dev = device()
    import torch
    wl = synth.by_name("fp8_qwen3_gateup_small")
    t = synth.make_fp8_inputs(wl, dev)

    def to_bytes(s):
        # E8M0 exponent bytes, the k-block dim padded to a multiple of 4
        # (four per int32 word)
        b = ((s.view(torch.int32) >> 23) & 0xFF).to(torch.uint8)
        g = b.shape[-1]
        pad = (-g) % 4
        if pad:
            b = torch.cat([b, torch.full((*b.shape[:-1], pad), 127, dtype=torch.uint8, device=dev)], -1)
        return b.contiguous()

    say("fp8 E8M0 byte scales")
    e = wl.num_groups
    y1 = sentinel_tensor((wl.m, wl.n), torch.bfloat16, dev)
    run_fp8(wl, t, y1)
    xs = gg.fp8_pack_scales(gg.GG_FP8_ACT_RAGGED, to_bytes(t["sx"]), t["offs"], wl.m, wl.k, e)
    ws = gg.fp8_pack_scales(gg.GG_FP8_WEIGHT, to_bytes(t["sw"]), None, wl.n, wl.k, e)
    y2 = sentinel_tensor((wl.m, wl.n), torch.bfloat16, dev)
    gg.fp8_forward(t["x8"], xs, t["w8"], ws, t["offs"], out=y2)
    torch.cuda.synchronize()
    assert np.array_equal(host(y1), host(y2))


def _sample_rows(wl, rng, count):
    """Rows to check: every expert's first and last active rows, rows at
    256-row tile boundaries, and random active rows (flat indices)."""
    sizes = wl.group_sizes()
    picks = []
    if wl.layout == "masked":
        for e in range(wl.num_groups):
            if sizes[e]:
                picks += [e * wl.m, e * wl.m + int(sizes[e]) - 1]
        active = np.concatenate([e * wl.m + np.arange(sizes[e]) for e in range(wl.num_groups)])
    else:
        ends = np.cumsum(sizes)
        starts = ends - sizes
        for s, e in zip(starts, ends):
            if e > s:
                picks += [int(s), int(e) - 1, int(min(s + 255, e - 1)), int(min(s + 256, e - 1))]
        active = np.arange(int(ends[-1]))
    picks += list(rng.choice(active, size=min(count, len(active)), replace=False))
    return np.unique(np.asarray(picks, dtype=np.int64))


@pytest.mark.parametrize("name,count", [("fp8_glm_up", 24)])
def test_fp8_forward_full_size_sampled(name, count):
    dev = device()
    import torch
    wl = synth.by_name(name)
    say("fp8 full-size", name, "drawing inputs")
    t = synth.make_fp8_inputs(wl, dev)
    y = torch.empty(out_shape(wl), dtype=torch.bfloat16, device=dev)
    say("fp8 full-size", name)
    run_fp8(wl, t, y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = _sample_rows(wl, rng, count)
    if name == "fp8_glm_up":
        rows = rows[rng.permutation(len(rows))[:96]]
    ref = oracle_fp8(wl, t, rows=rows)
    assert np.all(ref.status == 1)
    yh = host(y).reshape(-1, wl.n)[rows]
    rep = Report()
    check_fp8(yh, ref.value, ref.sabs, wl.k, f"fp8 {name} sampled", rep)
    print(name, len(rows), "rows", rep)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["fp8_qwen3_gateup", "fp8_masked_down", "fp8_masked_gateup"])
def test_fp8_forward_full_size_every_element(name):
    """The full-size Qwen3 gate/up shape (ragged) and the masked down and
    gate/up projections of the page's operand table, in the benchmark's
    launch configuration, compared element by element with the oracle in
    row chunks; rows outside the experts (inactive rows) keep the sentinel."""
    dev = device()
    import torch
    wl = synth.by_name(name)
    say("fp8 full-size every element", name, "drawing inputs")
    t = synth.make_fp8_inputs(wl, dev)
    y = sentinel_tensor(out_shape(wl), torch.bfloat16, dev)
    say("fp8 full-size every element", name)
    run_fp8(wl, t, y)
    torch.cuda.synchronize()
    yh = host(y).reshape(-1, wl.n)
    total = yh.shape[0]
    rep = Report()
    for r0 in range(0, total, 8192):
        rows = np.arange(r0, min(r0 + 8192, total))
        ref = oracle_fp8(wl, t, rows=rows)
        used = ref.status == 1
        g = yh[rows]
        check_fp8(g[used], ref.value[used], ref.sabs[used], wl.k, f"fp8 {name} rows {r0}..", rep)
        assert np.all(raw_bits(g[~used]) == sentinel_bits(y.dtype)), f"{name}: a row outside the experts was written"
    assert rep.n == int(wl.group_sizes().sum()) * wl.n
    print(name, rep)


@pytest.mark.parametrize("mm,max_m,k,n", [
    ([0, 300, 257, 1], 300, 128, 8),          # max_m not a multiple of 256: two row tiles per expert
    ([5, 0, 0, 129], 130, 256, 24),
])
def test_fp8_masked_edges(mm, max_m, k, n):
    dev = device()
    wl = synth.custom_masked("fp8_masked_edges", mm, max_m, k, n, seed=51 + k)
    t = synth.make_fp8_inputs(wl, dev)
    y = sentinel_tensor((wl.num_groups, wl.m, wl.n), _dt("bf16"), dev)
    say("fp8 masked edges", mm, max_m, k, n)
    run_fp8(wl, t, y)
    check_all_rows(wl, t, y, f"fp8 masked edges {mm} {max_m}")


def test_fp8_invalid_offsets_are_clamped():
    """Decreasing and oversize end offsets: the pack step and the GEMM clamp
    them the same way (end(g) = min(max(offs[0..g]), M)), so the result is
    the oracle's on the clamped grouping and no row past M is touched."""
    dev = device()
    import torch
    sizes = [40, 300, 9, 200]
    wl = synth.custom_ragged("fp8_bad_offs", sizes, 256, 136, seed=61, m=560)
    t = synth.make_fp8_inputs(wl, dev)
    bad = np.array([40, 20, 349, 10 ** 6], dtype=np.int32)      # decreasing, then past M
    t["offs"] = torch.from_numpy(bad).to(dev)
    wl.offs = bad
    y = sentinel_tensor((wl.m, wl.n), _dt("f32"), dev)
    say("fp8 invalid offsets")
    run_fp8(wl, t, y)
    check_all_rows(wl, t, y, "fp8 clamped offsets")
