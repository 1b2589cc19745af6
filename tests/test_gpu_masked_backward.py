"""GPU parity of the masked backward (gg_masked_dgrad, gg_masked_wgrad and
their scaled forms) against the oracle.  Inactive rows of dY and X hold NaN
(never read, so it must not reach any output); inactive rows of dX hold a
sentinel (never written); an expert with no active rows gets dW = +0."""
import numpy as np
import pytest

import oracle
from moe_grouped_gemm_ragged_amd import binding as gg
from moe_grouped_gemm_ragged_amd import synth
from gpu_util import device, host, raw_bits, say, sentinel_bits, sentinel_tensor
from parity import Report, check

pytestmark = pytest.mark.gpu

EDGE_MM = [0, 8, 256, 300, -3, 100, 1, 255, 129, 0]


def _dt(name):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _cases():
    return [synth.by_name("masked_down_small"),
            synth.custom_masked("masked_edge", EDGE_MM, 256, 264, 136, seed=17)]


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("case", [0, 1])
def test_masked_dgrad(case, out):
    import torch
    dev = device()
    wl = _cases()[case]
    t = synth.make_inputs(wl, dev, need=("w", "dy"))
    odt = _dt(out)
    dx = sentinel_tensor((wl.num_groups, wl.m, wl.k), odt, dev)
    say("masked dgrad", wl.name, out)
    gg.masked_dgrad(t["dy"], t["w"], t["masked_m"], out=dx)
    torch.cuda.synchronize()
    ref = oracle.masked_dgrad(synth.bf16_bits(t["dy"]), synth.bf16_bits(t["w"]), wl.masked_m)
    act = ref.status == 1
    dxh = host(dx).reshape(wl.num_groups * wl.m, wl.k)
    rep = Report()
    check(dxh[act], ref.value[act], ref.sabs[act], wl.n, "masked dgrad", rep)
    assert np.all(raw_bits(dxh[~act]) == sentinel_bits(odt)), "an inactive row was written"
    print(wl.name, out, rep)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("case", [0, 1])
def test_masked_wgrad(case, out):
    import torch
    dev = device()
    wl = _cases()[case]
    t = synth.make_inputs(wl, dev, need=("x", "dy"))
    odt = _dt(out)
    dw = sentinel_tensor((wl.num_groups, wl.k, wl.n), odt, dev)
    say("masked wgrad", wl.name, out)
    gg.masked_wgrad(t["x"], t["dy"], t["masked_m"], out=dw)
    torch.cuda.synchronize()
    ref = oracle.masked_wgrad(synth.bf16_bits(t["x"]), synth.bf16_bits(t["dy"]), wl.masked_m)
    dwh = host(dw).reshape(wl.num_groups * wl.k, wl.n)
    sizes = wl.group_sizes()
    L = np.repeat(np.maximum(sizes, 1), wl.k)[:, None]
    rep = Report()
    check(dwh, ref.value, ref.sabs, L, "masked wgrad", rep)
    empty = np.repeat(sizes == 0, wl.k)
    assert np.all(raw_bits(dwh[empty]) == 0), "an empty expert's dW is not +0.0"
    print(wl.name, out, rep, "empty:", int((sizes == 0).sum()))


@pytest.mark.parametrize("alpha,beta", [(1.0, 1.0), (-0.5, 2.0), (0.0, 1.0)])
def test_masked_backward_scaled(alpha, beta):
    import torch
    dev = device()
    wl = _cases()[1]
    t = synth.make_inputs(wl, dev, need=("x", "w", "dy"))
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    dx = (torch.randn((wl.num_groups, wl.m, wl.k), generator=g, device=dev) * 2).to(torch.bfloat16)
    dw = torch.randn((wl.num_groups, wl.k, wl.n), generator=g, device=dev) * 2
    cdx = host(dx).reshape(wl.num_groups * wl.m, wl.k)
    cdw = host(dw).reshape(wl.num_groups * wl.k, wl.n)
    say("masked backward scaled", alpha, beta)
    gg.masked_dgrad(t["dy"], t["w"], t["masked_m"], out=dx, alpha=alpha, beta=beta)
    gg.masked_wgrad(t["x"], t["dy"], t["masked_m"], out=dw, alpha=alpha, beta=beta)
    torch.cuda.synchronize()
    hx, hw, hdy = (synth.bf16_bits(t[k]) for k in ("x", "w", "dy"))
    rd = oracle.masked_dgrad(hdy, hw, wl.masked_m, alpha=alpha, beta=beta, c_in=cdx)
    act = rd.status == 1
    dxh = host(dx).reshape(wl.num_groups * wl.m, wl.k)
    check(dxh[act], rd.value[act], rd.sabs[act], wl.n + 1, "scaled masked dgrad")
    assert np.array_equal(dxh[~act], cdx[~act]), "an inactive row was touched"
    rw = oracle.masked_wgrad(hx, hdy, wl.masked_m, alpha=alpha, beta=beta, c_in=cdw)
    L = np.repeat(np.maximum(wl.group_sizes(), 1), wl.k)[:, None] + 1
    check(host(dw).reshape(-1, wl.n), rw.value, rw.sabs, L, "scaled masked wgrad")


@pytest.mark.timeout(600)
def test_masked_backward_full_size():
    """The masked down-projection workload (64 experts x 256 rows, K 768,
    N 2048), element by element: every active row of dX, with every
    inactive row still holding the sentinel, and all of dW."""
    import torch
    dev = device()
    wl = synth.masked_down()
    t = synth.make_inputs(wl, dev, need=("x", "w", "dy"))
    dx = sentinel_tensor((wl.num_groups, wl.m, wl.k), torch.bfloat16, dev)
    dw = sentinel_tensor((wl.num_groups, wl.k, wl.n), torch.float32, dev)
    say("full masked backward, every element")
    gg.masked_dgrad(t["dy"], t["w"], t["masked_m"], out=dx)
    gg.masked_wgrad(t["x"], t["dy"], t["masked_m"], out=dw)
    torch.cuda.synchronize()
    hx, hw, hdy = (synth.bf16_bits(t[k]) for k in ("x", "w", "dy"))
    rep = Report()
    rd = oracle.masked_dgrad(hdy, hw, wl.masked_m)
    act = rd.status == 1
    got = host(dx).reshape(-1, wl.k)
    check(got[act], rd.value[act], rd.sabs[act], wl.n, "full masked dgrad", rep)
    assert np.all(raw_bits(got[~act]) == synth.OUT_SENTINEL_BF16), "an inactive row was written"
    sizes = wl.group_sizes()
    rw = oracle.masked_wgrad(hx, hdy, wl.masked_m)
    got = host(dw).reshape(-1, wl.n)
    L = np.repeat(np.maximum(sizes, 1), wl.k)[:, None]
    check(got, rw.value, rw.sabs, L, "full masked wgrad", rep)
    empty = np.repeat(sizes == 0, wl.k)
    assert np.all(got[empty].view(np.uint32) == 0), "an empty expert's dW is not +0.0"
    print(rep)
