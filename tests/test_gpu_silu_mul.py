"""GPU parity of the gate/up forward with the fused SiLU-mul activation
(gg_forward_silu_mul, gg_masked_forward_silu_mul) against the oracle:
out = silu(G) * U on the gate and up halves of X . W13[g], one rounding.
Rows no expert owns (and inactive masked rows) must stay untouched; the
activation width I need not be a multiple of the 128-column output tile."""
import numpy as np
import pytest

import oracle
from moe_grouped_gemm_ragged_amd import binding as gg
from moe_grouped_gemm_ragged_amd import synth
from gpu_util import device, host, raw_bits, say, sentinel_bits, sentinel_tensor
from parity import Report, check

pytestmark = pytest.mark.gpu

SIZES = [0, 1, 7, 129, 0, 300, 16, 255, 0, 64]


def _dt(name):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("k,inter", [(264, 136), (136, 256), (2048, 768)])
def test_forward_silu_mul(k, inter, out):
    import torch
    dev = device()
    wl = synth.custom_ragged(f"silu_{k}_{inter}", SIZES, k, 2 * inter, seed=41 + inter,
                             m=int(sum(SIZES)) + 9, w_std=0.05)
    t = synth.make_inputs(wl, dev, need=("x", "w"))
    odt = _dt(out)
    a = sentinel_tensor((wl.m, inter), odt, dev)
    say("forward silu-mul", k, inter, out)
    gg.forward_silu_mul(t["x"], t["w"], t["offs"], out=a)
    torch.cuda.synchronize()
    ref = oracle.forward_silu_mul(synth.bf16_bits(t["x"]), synth.bf16_bits(t["w"]), wl.offs)
    ok = ref.status == 1
    ah = host(a)
    rep = Report()
    check(ah[ok], ref.value[ok], ref.sabs[ok], k, "silu-mul", rep)
    assert np.all(raw_bits(ah[~ok]) == sentinel_bits(odt)), "a row no expert owns was written"
    print(k, inter, out, rep)


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_masked_forward_silu_mul(out):
    import torch
    dev = device()
    mm = np.array([0, 8, 256, 300, -3, 100, 1, 255, 129, 0], dtype=np.int32)
    wl = synth.custom_masked("masked_silu", mm, 256, 264, 2 * 136, seed=43, w_std=0.05)
    t = synth.make_inputs(wl, dev, need=("x", "w"))
    odt = _dt(out)
    a = sentinel_tensor((wl.num_groups, wl.m, 136), odt, dev)
    say("masked silu-mul", out)
    gg.masked_forward_silu_mul(t["x"], t["w"], t["masked_m"], out=a)
    torch.cuda.synchronize()
    ref = oracle.masked_forward_silu_mul(synth.bf16_bits(t["x"]), synth.bf16_bits(t["w"]), mm)
    ok = ref.status == 1
    ah = host(a).reshape(wl.num_groups * wl.m, 136)
    rep = Report()
    check(ah[ok], ref.value[ok], ref.sabs[ok], wl.k, "masked silu-mul", rep)
    assert np.all(raw_bits(ah[~ok]) == sentinel_bits(odt)), "an inactive row was written"
    assert np.all(np.isfinite(ref.value[ok]))
    print(out, rep)


def test_silu_mul_equals_unfused_within_one_rounding():
    """The fused result against silu(G) * U computed by torch from the plain
    fp32 forward of the same problem (which rounds G and U to fp32 first)."""
    import torch
    dev = device()
    wl = synth.custom_ragged("silu_vs_unfused", SIZES, 264, 2 * 136, seed=44, w_std=0.05)
    t = synth.make_inputs(wl, dev, need=("x", "w"))
    say("silu-mul vs unfused")
    fused = gg.forward_silu_mul(t["x"], t["w"], t["offs"], out_dtype=torch.float32)
    h = gg.forward(t["x"], t["w"], t["offs"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    used = int(wl.offs[-1])
    ref = torch.nn.functional.silu(h[:used, :136].double()) * h[:used, 136:].double()
    err = (fused[:used].double() - ref).abs()
    assert float(err.max()) <= 1e-4 * max(1.0, float(ref.abs().max()))
