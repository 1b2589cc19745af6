"""GPU parity of the [E, N, K] weight-layout passes (gg_forward_nk,
gg_dgrad_nk, gg_wgrad_nk, gg_masked_forward_nk and their alpha/beta forms)
against the fp64 oracle, on the scaled-down workloads with every row,
sentinel-filled outputs (rows no expert owns stay untouched), both output
types, and the GLM-up shape on sampled rows.  Tolerance: parity.check."""
import numpy as np
import pytest

import oracle
from moe_grouped_gemm_ragged_amd import binding as gg
from moe_grouped_gemm_ragged_amd import synth
from gpu_util import device, host, raw_bits, say, sentinel_bits, sentinel_tensor
from parity import Report, check

pytestmark = pytest.mark.gpu

SMALL = ["tiny", "qwen3_gateup_small", "dsv3_small", "glm_up_small"]


def _dt(name):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def nk_inputs(wl, dev):
    t = synth.make_inputs(wl, dev)
    t["w_nk"] = t["w"].transpose(1, 2).contiguous()      # [E, N, K]
    return t


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("name", SMALL)
def test_forward_and_dgrad_nk_small(name, out):
    dev = device()
    import torch
    wl = synth.by_name(name)
    t = nk_inputs(wl, dev)
    y = sentinel_tensor((wl.m, wl.n), _dt(out), dev)
    dx = sentinel_tensor((wl.m, wl.k), _dt(out), dev)
    say("forward_nk / dgrad_nk", name, out)
    gg.forward_nk(t["x"], t["w_nk"], t["offs"], out=y)
    gg.dgrad_nk(t["dy"], t["w_nk"], t["offs"], out=dx)
    torch.cuda.synchronize()
    wnk = synth.bf16_bits(t["w_nk"])
    rf = oracle.forward_nk(synth.bf16_bits(t["x"]), wnk, wl.offs)
    rd = oracle.dgrad_nk(synth.bf16_bits(t["dy"]), wnk, wl.offs)
    used = rf.status == 1
    rep = Report()
    yh, dh = host(y), host(dx)
    check(yh[used], rf.value[used], rf.sabs[used], wl.k, f"forward_nk {name}", rep)
    check(dh[used], rd.value[used], rd.sabs[used], wl.n, f"dgrad_nk {name}", rep)
    assert np.all(raw_bits(yh[~used]) == sentinel_bits(_dt(out)))
    assert np.all(raw_bits(dh[~used]) == sentinel_bits(_dt(out)))
    print(name, out, rep)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("name", SMALL)
def test_wgrad_nk_small(name, out):
    dev = device()
    import torch
    wl = synth.by_name(name)
    t = nk_inputs(wl, dev)
    dw = sentinel_tensor((wl.num_groups, wl.n, wl.k), _dt(out), dev)
    say("wgrad_nk", name, out)
    gg.wgrad_nk(t["x"], t["dy"], t["offs"], out=dw)
    torch.cuda.synchronize()
    ref = oracle.wgrad_nk(synth.bf16_bits(t["x"]), synth.bf16_bits(t["dy"]), wl.offs)
    L = np.repeat(np.maximum(wl.group_sizes(), 1), wl.n)[:, None]
    rep = Report()
    check(host(dw).reshape(-1, wl.k), ref.value, ref.sabs, L, f"wgrad_nk {name}", rep)
    print(name, out, rep)


def test_masked_forward_nk_small():
    dev = device()
    import torch
    wl = synth.by_name("masked_down_small")
    t = synth.make_inputs(wl, dev, need=("x", "w"))
    w_nk = t["w"].transpose(1, 2).contiguous()
    y = sentinel_tensor((wl.num_groups, wl.m, wl.n), torch.bfloat16, dev)
    say("masked_forward_nk")
    gg.masked_forward_nk(t["x"], w_nk, t["masked_m"], out=y)
    torch.cuda.synchronize()
    ref = oracle.masked_forward_nk(synth.bf16_bits(t["x"]), synth.bf16_bits(w_nk), wl.masked_m)
    yh = host(y).reshape(-1, wl.n)
    act = ref.status == 1
    check(yh[act], ref.value[act], ref.sabs[act], wl.k, "masked_forward_nk")
    assert np.all(raw_bits(yh[~act]) == sentinel_bits(torch.bfloat16))


def test_nk_agrees_with_kn_layout():
    """The same product in either weight layout (fp32 outputs; the reduction
    order may differ, so within 1e-5 of the largest value), and the alpha /
    beta form of the [E, N, K] forward accumulates into its output."""
    dev = device()
    import torch
    wl = synth.by_name("qwen3_gateup_small")
    t = nk_inputs(wl, dev)
    y1 = gg.forward(t["x"], t["w"], t["offs"], out_dtype=torch.float32)
    y2 = gg.forward_nk(t["x"], t["w_nk"], t["offs"], out_dtype=torch.float32)
    y3 = y2.clone()
    gg.forward_nk(t["x"], t["w_nk"], t["offs"], out=y3, alpha=0.5, beta=1.0)
    torch.cuda.synchronize()
    used = int(wl.offs[-1])
    a, b, c = (v[:used].cpu().numpy().astype(np.float64) for v in (y1, y2, y3))
    scale = np.abs(a).max()
    assert np.max(np.abs(a - b)) <= 1e-5 * scale
    assert np.max(np.abs(c - 1.5 * b)) <= 1e-5 * scale


def test_glm_up_nk_sampled():
    dev = device()
    import torch
    wl = synth.glm_up()
    say("glm_up nk drawing")
    t = nk_inputs(wl, dev)
    del t["w"]
    y = torch.empty((wl.m, wl.n), dtype=torch.bfloat16, device=dev)
    say("glm_up forward_nk")
    gg.forward_nk(t["x"], t["w_nk"], t["offs"], out=y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.choice(wl.m, 40, replace=False), wl.offs[:8] - 1, [0]]))
    ref = oracle.forward_nk(synth.bf16_bits(t["x"]), synth.bf16_bits(t["w_nk"]), wl.offs, rows=rows)
    check(host(y)[rows], ref.value, ref.sabs, wl.k, "glm_up forward_nk sampled")
