"""GPU parity of the grouped bias with a per-token factor (gg_forward_bias,
gg_masked_forward_bias) against the fp64 oracle:
* ragged workloads with unused capacity rows (sentinel-filled, must stay
  untouched) and a factor array holding exactly the logical rows, bf16 and
  fp32 outputs, with and without the factor, with alpha / beta;
* the masked layout with NaN factors and NaN rows in the inactive region;
* the bias entry point with a zero bias and no factor equals the plain
  forward bit for bit.
Tolerance: parity.check."""
import numpy as np
import pytest

import oracle
from moe_grouped_gemm_ragged_amd import binding as gg
from moe_grouped_gemm_ragged_amd import synth
from gpu_util import device, host, raw_bits, say, sentinel_bits, sentinel_tensor
from parity import Report, check

pytestmark = pytest.mark.gpu


def _dt(name):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def draws(wl, dev, logical):
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed * 7919 + 5)
    bias = (torch.randn((wl.num_groups, wl.n), generator=g, device=dev) * 0.5).to(torch.bfloat16)
    scale = torch.rand((logical,), generator=g, device=dev, dtype=torch.float32)
    return bias, scale


@pytest.mark.parametrize("with_scale", [True, False])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("name,capacity", [("qwen3_gateup_small", 37), ("dsv3_small", 0), ("tiny", 5)])
def test_forward_bias_ragged(name, capacity, out, with_scale):
    dev = device()
    import torch
    base = synth.by_name(name)
    sizes = base.group_sizes()
    wl = synth.custom_ragged(name + "_cap", sizes, base.k, base.n, seed=base.seed,
                             m=int(base.offs[-1]) + capacity + (base.m - int(base.offs[-1])))
    t = synth.make_inputs(wl, dev)
    logical = int(wl.offs[-1])
    bias, scale = draws(wl, dev, logical)
    bs = scale if with_scale else None
    y = sentinel_tensor((wl.m, wl.n), _dt(out), dev)
    say("forward_bias", name, out, with_scale)
    gg.forward_bias(t["x"], t["w"], t["offs"], bias, bs, out=y)
    torch.cuda.synchronize()
    ref = oracle.forward_bias(synth.bf16_bits(t["x"]), synth.bf16_bits(t["w"]), wl.offs,
                              synth.bf16_bits(bias), None if bs is None else bs.cpu().numpy())
    yh = host(y)
    used = ref.status == 1
    rep = Report()
    check(yh[used], ref.value[used], ref.sabs[used], wl.k + 1, f"forward_bias {name}", rep)
    assert np.all(raw_bits(yh[~used]) == sentinel_bits(_dt(out))), "capacity rows were written"
    print(name, out, with_scale, rep)


def test_forward_bias_alpha_beta():
    dev = device()
    import torch
    wl = synth.by_name("glm_up_small")
    t = synth.make_inputs(wl, dev)
    bias, scale = draws(wl, dev, int(wl.offs[-1]))
    y = torch.randn((wl.m, wl.n), device=dev, dtype=torch.float32)
    c0 = y.cpu().numpy().copy()
    say("forward_bias alpha/beta")
    gg.forward_bias(t["x"], t["w"], t["offs"], bias, scale, out=y, alpha=0.75, beta=-0.5)
    torch.cuda.synchronize()
    ref = oracle.forward_bias(synth.bf16_bits(t["x"]), synth.bf16_bits(t["w"]), wl.offs,
                              synth.bf16_bits(bias), scale.cpu().numpy(), alpha=0.75, beta=-0.5, c_in=c0)
    used = ref.status == 1
    check(host(y)[used], ref.value[used], ref.sabs[used], wl.k + 2, "forward_bias alpha/beta")


def test_masked_forward_bias_inactive_factors_not_read():
    dev = device()
    import torch
    wl = synth.by_name("masked_down_small")
    t = synth.make_inputs(wl, dev, need=("x", "w"))
    bias, _ = draws(wl, dev, 1)
    scale = torch.rand((wl.num_groups, wl.m), device=dev, dtype=torch.float32)
    sizes = wl.group_sizes()
    for e in range(wl.num_groups):
        scale[e, int(sizes[e]):] = float("nan")
    y = sentinel_tensor((wl.num_groups, wl.m, wl.n), torch.bfloat16, dev)
    say("masked_forward_bias")
    gg.masked_forward_bias(t["x"], t["w"], t["masked_m"], bias, scale, out=y)
    torch.cuda.synchronize()
    ref = oracle.masked_forward_bias(synth.bf16_bits(t["x"]), synth.bf16_bits(t["w"]), wl.masked_m,
                                     synth.bf16_bits(bias), scale.cpu().numpy())
    yh = host(y).reshape(-1, wl.n)
    act = ref.status == 1
    check(yh[act], ref.value[act], ref.sabs[act], wl.k + 1, "masked_forward_bias")
    assert np.all(raw_bits(yh[~act]) == sentinel_bits(torch.bfloat16))


def test_zero_bias_equals_plain_forward():
    dev = device()
    import torch
    wl = synth.by_name("qwen3_gateup_small")
    t = synth.make_inputs(wl, dev)
    zero = torch.zeros((wl.num_groups, wl.n), dtype=torch.bfloat16, device=dev)
    y1 = gg.forward(t["x"], t["w"], t["offs"])
    y2 = gg.forward_bias(t["x"], t["w"], t["offs"], zero, None)
    torch.cuda.synchronize()
    used = int(wl.offs[-1])
    assert np.array_equal(host(y1)[:used], host(y2)[:used])


@pytest.mark.parametrize("with_scale", [True, False])
def test_bias_grad_ragged_with_capacity(with_scale):
    dev = device()
    import torch
    base = synth.by_name("dsv3_small")
    wl = synth.custom_ragged("dbias", base.group_sizes(), base.k, base.n, seed=3, m=int(base.offs[-1]) + 29)
    t = synth.make_inputs(wl, dev, need=("dy",))
    logical = int(wl.offs[-1])
    scale = torch.rand((logical,), device=dev) if with_scale else None
    say("bias_grad", with_scale)
    db = gg.bias_grad(t["dy"], t["offs"], scale)
    torch.cuda.synchronize()
    ref = oracle.bias_grad(synth.bf16_bits(t["dy"]), wl.offs, None if scale is None else scale.cpu().numpy())
    L = int(max(1, wl.group_sizes().max()))
    check(db.cpu().numpy(), ref.value, ref.sabs, L, "bias_grad")
    empty = np.flatnonzero(wl.group_sizes() == 0)
    assert np.all(db.cpu().numpy()[empty] == 0.0)


def test_bias_scale_grad_ragged_and_masked():
    dev = device()
    import torch
    wl = synth.by_name("qwen3_gateup_small")
    t = synth.make_inputs(wl, dev, need=("dy",))
    bias = (torch.randn((wl.num_groups, wl.n), device=dev) * 0.5).to(torch.bfloat16)
    say("bias_scale_grad ragged")
    ds = gg.bias_scale_grad(t["dy"], t["offs"], bias)
    torch.cuda.synchronize()
    ref = oracle.bias_scale_grad(synth.bf16_bits(t["dy"]), wl.offs, synth.bf16_bits(bias))
    ok = ref.status == 1
    dh = ds.cpu().numpy()
    check(dh[ok][:, None], ref.value[ok], ref.sabs[ok], wl.n, "bias_scale_grad")
    assert np.all(np.isnan(dh[~ok])), "rows no expert owns were written"
    wm = synth.by_name("masked_down_small")
    tm = synth.make_inputs(wm, dev, need=("dy",))
    bm = (torch.randn((wm.num_groups, wm.n), device=dev) * 0.5).to(torch.bfloat16)
    say("bias grads masked")
    dsm = gg.bias_scale_grad(tm["dy"], tm["masked_m"], bm, masked=True)
    dbm = gg.bias_grad(tm["dy"], tm["masked_m"], None, masked=True)
    torch.cuda.synchronize()
    rm = oracle.bias_scale_grad(synth.bf16_bits(tm["dy"]), wm.masked_m, synth.bf16_bits(bm), masked=True)
    okm = rm.status == 1
    dmh = dsm.cpu().numpy()
    check(dmh[okm][:, None], rm.value[okm], rm.sabs[okm], wm.n, "masked bias_scale_grad")
    assert np.all(np.isnan(dmh[~okm]))
    rb = oracle.bias_grad(synth.bf16_bits(tm["dy"]), wm.masked_m, None, masked=True)
    check(dbm.cpu().numpy(), rb.value, rb.sabs, wm.m, "masked bias_grad")


def test_bias_grads_clamped_offsets_many_experts_partial_columns():
    """600 experts (more offsets than a workgroup has threads), N = 200 (a
    partial 128-column block), empty experts, and offsets that decrease, go
    negative or pass M (clamped as everywhere).  Both reductions must match
    the oracle, repeat bit for bit, give +0.0 for every empty expert and
    leave rows no expert owns untouched."""
    import torch
    dev = device()
    rng = np.random.default_rng(11)
    e, n = 600, 200
    sizes = rng.integers(0, 12, size=e)
    sizes[::7] = 0
    m = int(sizes.sum()) + 13
    wl = synth.custom_ragged("dbias_many", sizes, 8, n, seed=5, m=m)
    t = synth.make_inputs(wl, dev, need=("dy",))
    offs_h = wl.offs.astype(np.int32).copy()
    offs_h[5] = offs_h[4] - 3          # decreasing: expert 5 is empty
    offs_h[9] = -4                     # negative: expert 9 is empty
    offs_h[e - 2] = m + 50             # past M: expert e-2 runs to M, expert e-1 is empty
    offs = torch.tensor(offs_h, dtype=torch.int32, device=dev)
    scale = torch.rand((m,), device=dev)
    bias = (torch.randn((e, n), device=dev) * 0.5).to(torch.bfloat16)
    say("bias grads, 600 experts, clamped offsets, n 200")
    db1 = gg.bias_grad(t["dy"], offs, scale)
    db2 = gg.bias_grad(t["dy"], offs, scale)
    ds1 = gg.bias_scale_grad(t["dy"], offs, bias)
    ds2 = gg.bias_scale_grad(t["dy"], offs, bias)
    torch.cuda.synchronize()
    assert torch.equal(db1.view(torch.int32), db2.view(torch.int32)), "dbias not repeatable"
    assert torch.equal(ds1.view(torch.int32), ds2.view(torch.int32)), "dscale not repeatable"
    dy_bits = synth.bf16_bits(t["dy"])
    ref = oracle.bias_grad(dy_bits, offs_h, scale.cpu().numpy())
    ends = np.minimum(np.maximum.accumulate(np.maximum(offs_h.astype(np.int64), 0)), m)
    rows = np.diff(np.concatenate([[0], ends]))
    check(db1.cpu().numpy(), ref.value, ref.sabs, int(max(1, rows.max())), "bias_grad clamped")
    assert np.all(db1.cpu().numpy()[rows == 0] == 0.0) and not np.any(np.signbit(db1.cpu().numpy()[rows == 0]))
    rs = oracle.bias_scale_grad(dy_bits, offs_h, synth.bf16_bits(bias))
    ok = rs.status == 1
    dh = ds1.cpu().numpy()
    check(dh[ok][:, None], rs.value[ok], rs.sabs[ok], n, "bias_scale_grad clamped")
    assert np.all(np.isnan(dh[~ok])), "rows no expert owns were written"


def test_masked_bias_grads_out_of_range_counts_partial_columns():
    """Masked layout with counts below 0 and above max_m (clamped) and
    N = 136: dbias over the active rows only, ds only on active rows."""
    import torch
    dev = device()
    rng = np.random.default_rng(12)
    e, max_m, n = 300, 40, 136
    mm = rng.integers(0, max_m + 1, size=e).astype(np.int32)
    mm[3], mm[4], mm[5] = -7, max_m + 9, 0
    wl = synth.custom_masked("dbias_masked", mm, max_m, 8, n, seed=6)
    t = synth.make_inputs(wl, dev, need=("dy",))
    counts = torch.tensor(mm, dtype=torch.int32, device=dev)
    scale = torch.rand((e * max_m,), device=dev)
    bias = (torch.randn((e, n), device=dev) * 0.5).to(torch.bfloat16)
    say("masked bias grads, out-of-range counts, n 136")
    db = gg.bias_grad(t["dy"], counts, scale, masked=True)
    ds = gg.bias_scale_grad(t["dy"], counts, bias, masked=True)
    torch.cuda.synchronize()
    dy_bits = synth.bf16_bits(t["dy"])
    ref = oracle.bias_grad(dy_bits, mm, scale.cpu().numpy(), masked=True)
    check(db.cpu().numpy(), ref.value, ref.sabs, max_m, "masked bias_grad clamped")
    active = np.clip(mm, 0, max_m)
    assert np.all(db.cpu().numpy()[active == 0] == 0.0)
    rs = oracle.bias_scale_grad(dy_bits, mm, synth.bf16_bits(bias), masked=True)
    ok = rs.status == 1
    dh = ds.cpu().numpy()
    check(dh[ok][:, None], rs.value[ok], rs.sabs[ok], n, "masked bias_scale_grad clamped")
    assert np.all(np.isnan(dh[~ok]))


def test_bias_grads_full_size_qwen3():
    """Both reductions at the Qwen3 gate/up size (65536 rows, N 1536, 128
    experts with empty and 8- / 16-row experts), against the oracle on every
    element."""
    import torch
    dev = device()
    wl = synth.by_name("qwen3_gateup")
    t = synth.make_inputs(wl, dev, need=("dy",))
    logical = int(wl.offs[-1])
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    scale = torch.rand((logical,), generator=g, device=dev)
    bias = (torch.randn((wl.num_groups, wl.n), generator=g, device=dev) * 0.5).to(torch.bfloat16)
    say("bias grads, qwen3_gateup full size")
    db = gg.bias_grad(t["dy"], t["offs"], scale)
    ds = gg.bias_scale_grad(t["dy"], t["offs"], bias)
    torch.cuda.synchronize()
    dy_bits = synth.bf16_bits(t["dy"])
    ref = oracle.bias_grad(dy_bits, wl.offs, scale.cpu().numpy())
    check(db.cpu().numpy(), ref.value, ref.sabs, int(wl.group_sizes().max()), "bias_grad qwen3")
    rs = oracle.bias_scale_grad(dy_bits, wl.offs, synth.bf16_bits(bias))
    ok = rs.status == 1
    check(ds.cpu().numpy()[ok][:, None], rs.value[ok], rs.sabs[ok], wl.n, "bias_scale_grad qwen3")


@pytest.mark.parametrize("masked", [False, True])
def test_bias_grads_large_experts_partial_columns(masked):
    """Experts of 1500-3000 rows (at least 2048 per expert on average, so
    workgroups take 128 columns) with N = 200 / 136, a partial block."""
    import torch
    dev = device()
    if masked:
        wl = synth.custom_masked("dbias_wide_masked", [2100, 1234], 2100, 8, 136, seed=8)
        groups_h = wl.masked_m
    else:
        wl = synth.custom_ragged("dbias_wide", [2048, 3000, 1500], 8, 200, seed=9, m=6548 + 100)
        groups_h = wl.offs
    t = synth.make_inputs(wl, dev, need=("dy",))
    groups = t["masked_m"] if masked else t["offs"]
    rows_total = wl.num_groups * wl.m if masked else wl.m
    scale = torch.rand((rows_total,), device=dev)
    say("bias grads, large experts", masked)
    db = gg.bias_grad(t["dy"], groups, scale, masked=masked)
    torch.cuda.synchronize()
    ref = oracle.bias_grad(synth.bf16_bits(t["dy"]), groups_h, scale.cpu().numpy(), masked=masked)
    check(db.cpu().numpy(), ref.value, ref.sabs, 3000, "bias_grad large experts")
