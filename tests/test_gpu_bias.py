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
