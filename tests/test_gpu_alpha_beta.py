"""GPU parity of the scaled and accumulating forms (gg_*_ex):
out = alpha * product + beta * out, combined in fp32 before the one rounding
(fused accumulation; TransformerEngine PR #3542, "Changes"), against the
oracle's fp64 alpha * P + beta * C on the same prior output.

Rows no expert owns (and inactive masked rows) must stay untouched; beta = 0
must not read the output (NaN in it is overwritten); accumulating wgrad must
leave an empty expert's dW bit-identical.
"""
import numpy as np
import pytest

import oracle
from moe_grouped_gemm_ragged_amd import binding as gg
from moe_grouped_gemm_ragged_amd import synth
from gpu_util import device, host, raw_bits, say, sentinel_bits
from parity import Report, check

pytestmark = pytest.mark.gpu

AB = [(1.0, 1.0), (-0.5, 2.0), (0.25, -1.0), (2.0, 0.0), (0.0, 1.0)]
SIZES = [0, 1, 7, 129, 0, 300, 16, 255, 0]


def _prior(shape, dtype, dev, used_rows=None, seed=0):
    """Finite random prior output; rows at or past used_rows hold the
    sentinel (they must come back untouched)."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(1234 + seed)
    t = (torch.randn(shape, generator=g, device=dev) * 3).to(dtype)
    if used_rows is not None:
        if dtype == torch.bfloat16:
            t.view(torch.int16)[used_rows:] = int(np.array([synth.OUT_SENTINEL_BF16], np.uint16).view(np.int16)[0])
        else:
            t.view(torch.int32)[used_rows:] = int(np.array([synth.OUT_SENTINEL_F32], np.uint32).view(np.int32)[0])
    return t


def _dt(name):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("alpha,beta", AB)
def test_scaled_ragged_passes(alpha, beta, out):
    import torch
    dev = device()
    wl = synth.custom_ragged("ab", SIZES, 264, 136, seed=91, m=int(sum(SIZES)) + 20)
    t = synth.make_inputs(wl, dev)
    used = int(wl.offs[-1])
    odt = _dt(out)
    y = _prior((wl.m, wl.n), odt, dev, used, seed=1)
    dx = _prior((wl.m, wl.k), odt, dev, used, seed=2)
    dw = _prior((wl.num_groups, wl.k, wl.n), torch.float32 if out == "f32" else torch.bfloat16, dev, seed=3)
    cy, cdx, cdw = host(y), host(dx), host(dw).reshape(wl.num_groups * wl.k, wl.n)
    say("scaled passes", alpha, beta, out)
    gg.forward(t["x"], t["w"], t["offs"], out=y, alpha=alpha, beta=beta)
    gg.dgrad(t["dy"], t["w"], t["offs"], out=dx, alpha=alpha, beta=beta)
    gg.wgrad(t["x"], t["dy"], t["offs"], out=dw, alpha=alpha, beta=beta)
    torch.cuda.synchronize()
    hx, hw, hdy = (synth.bf16_bits(t[k]) for k in ("x", "w", "dy"))
    rep = Report()
    rf = oracle.forward(hx, hw, wl.offs, alpha=alpha, beta=beta, c_in=cy)
    ok = rf.status == 1
    yh = host(y)
    check(yh[ok], rf.value[ok], rf.sabs[ok], wl.k + 1, "scaled fwd", rep)
    assert np.all(raw_bits(yh[~ok]) == sentinel_bits(odt)), "fwd touched a row no expert owns"
    rd = oracle.dgrad(hdy, hw, wl.offs, alpha=alpha, beta=beta, c_in=cdx)
    dxh = host(dx)
    check(dxh[ok], rd.value[ok], rd.sabs[ok], wl.n + 1, "scaled dgrad", rep)
    assert np.all(raw_bits(dxh[~ok]) == sentinel_bits(odt)), "dgrad touched a row no expert owns"
    rw = oracle.wgrad(hx, hdy, wl.offs, alpha=alpha, beta=beta, c_in=cdw)
    dwh = host(dw).reshape(wl.num_groups * wl.k, wl.n)
    sizes = wl.group_sizes()
    L = np.repeat(np.maximum(sizes, 1), wl.k)[:, None] + 1
    check(dwh, rw.value, rw.sabs, L, "scaled wgrad", rep)
    print(alpha, beta, out, rep)


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("alpha,beta", AB)
def test_scaled_masked(alpha, beta, out):
    import torch
    dev = device()
    mm = np.array([0, 8, 256, 100, 1, 129, 200, 0], dtype=np.int32)
    wl = synth.custom_masked("abm", mm, 256, 264, 136, seed=92)
    t = synth.make_inputs(wl, dev, need=("x", "w"))
    odt = _dt(out)
    y = _prior((wl.num_groups, wl.m, wl.n), odt, dev, seed=4)
    flat = y.view(wl.num_groups * wl.m, wl.n)
    act = np.zeros(wl.num_groups * wl.m, dtype=bool)
    for e, a in enumerate(mm):
        act[e * wl.m:e * wl.m + a] = True
    sent = torch.from_numpy(np.nonzero(~act)[0]).to(dev)
    if odt == torch.bfloat16:
        flat.view(torch.int16)[sent] = int(np.array([synth.OUT_SENTINEL_BF16], np.uint16).view(np.int16)[0])
    else:
        flat.view(torch.int32)[sent] = int(np.array([synth.OUT_SENTINEL_F32], np.uint32).view(np.int32)[0])
    cy = host(flat)
    say("scaled masked", alpha, beta, out)
    gg.masked_forward(t["x"], t["w"], t["masked_m"], out=y, alpha=alpha, beta=beta)
    torch.cuda.synchronize()
    ref = oracle.masked_forward(synth.bf16_bits(t["x"]), synth.bf16_bits(t["w"]), mm,
                                alpha=alpha, beta=beta, c_in=cy)
    ok = ref.status == 1
    assert np.array_equal(ok, act)
    yh = host(y).reshape(wl.num_groups * wl.m, wl.n)
    check(yh[ok], ref.value[ok], ref.sabs[ok], wl.k + 1, "scaled masked")
    assert np.all(raw_bits(yh[~ok]) == sentinel_bits(odt)), "an inactive row was touched"


def test_accumulating_wgrad_keeps_empty_experts_exactly():
    import torch
    dev = device()
    wl = synth.custom_ragged("acc", SIZES, 136, 264, seed=93)
    t = synth.make_inputs(wl, dev)
    dw = _prior((wl.num_groups, wl.k, wl.n), torch.float32, dev, seed=5)
    before = dw.clone()
    say("accumulate wgrad, empty experts")
    gg.wgrad(t["x"], t["dy"], t["offs"], out=dw, beta=1.0)
    torch.cuda.synchronize()
    for g, s in enumerate(wl.group_sizes()):
        if s == 0:
            assert torch.equal(dw[g].view(torch.int32), before[g].view(torch.int32))


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_beta_zero_overwrites_nan(out):
    """alpha = 2, beta = 0: the output is not read -- NaN in it is replaced,
    and the result is exactly twice the plain pass (scaling by two is exact)."""
    import torch
    dev = device()
    wl = synth.custom_ragged("b0", SIZES, 264, 136, seed=94)
    t = synth.make_inputs(wl, dev)
    odt = _dt(out)
    y = torch.full((wl.m, wl.n), float("nan"), dtype=odt, device=dev)
    say("beta 0 over NaN", out)
    gg.forward(t["x"], t["w"], t["offs"], out=y, alpha=2.0, beta=0.0)
    plain = gg.forward(t["x"], t["w"], t["offs"], out_dtype=odt)
    torch.cuda.synchronize()
    assert torch.equal(y, plain * 2)
