"""Graph capture: the three passes captured once in a HIP graph (through
torch.cuda.graph) keep following the offsets the device holds at replay
time.  The offsets tensor is rewritten in place between replays, with other
eager work and synchronisations in between, and every replay is compared
bit for bit with an eager call on the same offsets (the kernels are
deterministic) and, once, with the oracle.  This shows the library reads
the grouping on the device only, with no host copy baked into the graph."""
import numpy as np
import pytest

import oracle
from moe_grouped_gemm_ragged_amd import binding as gg
from moe_grouped_gemm_ragged_amd import synth
from gpu_util import device, host, say
from parity import check

pytestmark = pytest.mark.gpu


def test_graph_replay_follows_device_offsets():
    import torch
    dev = device()
    E, k, n = 12, 264, 520
    rng = np.random.default_rng(77)
    groupings = []
    for _ in range(4):
        sizes = rng.multinomial(1500, rng.dirichlet(np.ones(E)))
        sizes[rng.integers(0, E, 2)] = 0
        groupings.append(np.cumsum(sizes).astype(np.int32))
    m = int(max(g[-1] for g in groupings)) + 16
    wl = synth.Workload("graph", "ragged", E, m, k, n, seed=21, offs=groupings[0])
    t = synth.make_inputs(wl, dev)
    offs = t["offs"]
    y = torch.zeros((m, n), dtype=torch.bfloat16, device=dev)
    dx = torch.zeros((m, k), dtype=torch.bfloat16, device=dev)
    dw = torch.zeros((E, k, n), dtype=torch.float32, device=dev)

    def passes(yo, dxo, dwo):
        gg.forward(t["x"], t["w"], offs, out=yo)
        gg.dgrad(t["dy"], t["w"], offs, out=dxo)
        gg.wgrad(t["x"], t["dy"], offs, out=dwo)

    say("graph: warm-up and capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        passes(y, dx, dw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        passes(y, dx, dw)
    torch.cuda.synchronize()

    ye = torch.empty_like(y)
    dxe = torch.empty_like(dx)
    dwe = torch.empty_like(dw)
    for rep, new in enumerate(groupings[1:] + groupings[:1]):
        offs.copy_(torch.from_numpy(new).to(dev))     # in place, on the device
        y.fill_(0)
        dx.fill_(0)
        dw.fill_(float("nan"))
        say("graph replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        # other eager work between replays
        junk = torch.randn(512, 512, device=dev) @ torch.randn(512, 512, device=dev)
        ye.fill_(0)
        dxe.fill_(0)
        passes(ye, dxe, dwe)
        torch.cuda.synchronize()
        used = int(new[-1])
        assert torch.equal(y[:used], ye[:used]), f"replay {rep}: Y differs from eager"
        assert torch.equal(dx[:used], dxe[:used]), f"replay {rep}: dX differs from eager"
        assert torch.equal(dw, dwe), f"replay {rep}: dW differs from eager"
        assert bool(torch.all(y[used:] == 0)), f"replay {rep}: wrote past the last offset"
        del junk
        if rep == 0:
            hx, hw = synth.bf16_bits(t["x"]), synth.bf16_bits(t["w"])
            rf = oracle.forward(hx, hw, new)
            ok = rf.status == 1
            check(host(y)[ok], rf.value[ok], rf.sabs[ok], k, "graph fwd vs oracle")


def test_graph_replay_fp8_and_bias_paths():
    """The fp8 path (activation-scale packing, then the fp8 forward) and the
    grouped bias (forward with a per-token factor, then both bias gradients)
    captured in one graph.  Between replays the offsets and the fp8
    activation scales change in place on the device; every replay must equal
    an eager run of the same calls bit for bit, and the bad-scale counter
    (zeroed by a fill kernel inside the graph) must count afresh."""
    import torch
    dev = device()
    E, k, n = 6, 256, 264
    rng = np.random.default_rng(78)
    groupings = []
    for _ in range(3):
        sizes = rng.multinomial(900, rng.dirichlet(np.ones(E)))
        sizes[rng.integers(0, E)] = 0
        groupings.append(np.cumsum(sizes).astype(np.int32))
    m = int(max(g[-1] for g in groupings)) + 8
    wl = synth.Workload("graph8", "ragged", E, m, k, n, seed=22, offs=groupings[0])
    t8 = synth.make_fp8_inputs(wl, dev)
    t = synth.make_inputs(wl, dev)
    offs = t8["offs"]
    sx = t8["sx"]
    xs = torch.empty(gg.fp8_scale_bytes(gg.GG_FP8_ACT_RAGGED, m, k, E), dtype=torch.uint8, device=dev)
    ws = gg.fp8_pack_scales(gg.GG_FP8_WEIGHT, t8["sw"], None, n, k, E)
    bad = torch.zeros(1, dtype=torch.int32, device=dev)
    bias = (torch.randn((E, n), device=dev) * 0.5).to(torch.bfloat16)
    bscale = torch.rand((m,), device=dev)
    y8 = torch.zeros((m, n), dtype=torch.bfloat16, device=dev)
    yb = torch.zeros((m, n), dtype=torch.float32, device=dev)
    db = torch.zeros((E, n), dtype=torch.float32, device=dev)
    ds = torch.zeros((m,), dtype=torch.float32, device=dev)

    def calls(y8o, ybo, dbo, dso, bado):
        bado.zero_()
        gg.fp8_pack_scales(gg.GG_FP8_ACT_RAGGED, sx, offs, m, k, E, out=xs, bad_count=bado)
        gg.fp8_forward(t8["x8"], xs, t8["w8"], ws, offs, out=y8o)
        gg.forward_bias(t["x"], t["w"], offs, bias, bscale, out=ybo)
        gg.bias_grad(t["dy"], offs, bscale, out=dbo)
        gg.bias_scale_grad(t["dy"], offs, bias, out=dso)

    say("graph fp8 + bias: warm-up and capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls(y8, yb, db, ds, bad)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(y8, yb, db, ds, bad)
    torch.cuda.synchronize()

    y8e, ybe, dbe, dse = (torch.zeros_like(a) for a in (y8, yb, db, ds))
    bade = torch.zeros_like(bad)
    for rep, new in enumerate(groupings[1:] + groupings[:1]):
        offs.copy_(torch.from_numpy(new).to(dev))
        sx[0, 0] = 0.3 if rep % 2 == 0 else 1.0       # a non-UE8M0 scale in row 0 on even replays
        torch.cuda.synchronize()
        say("graph fp8 + bias replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.randn(256, 256, device=dev) @ torch.randn(256, 256, device=dev)
        calls(y8e, ybe, dbe, dse, bade)
        torch.cuda.synchronize()
        used = int(new[-1])
        assert torch.equal(y8[:used].view(torch.int16), y8e[:used].view(torch.int16)), f"replay {rep}: fp8 Y"
        assert torch.equal(yb[:used], ybe[:used]), f"replay {rep}: biased Y"
        assert torch.equal(db, dbe), f"replay {rep}: dbias"
        assert torch.equal(ds[:used], dse[:used]), f"replay {rep}: ds"
        want_bad = 1 if (rep % 2 == 0 and used > 0) else 0     # row 0 belongs to the first non-empty expert
        assert int(bad.item()) == int(bade.item()) == want_bad, f"replay {rep}: bad-scale count"
        del junk
