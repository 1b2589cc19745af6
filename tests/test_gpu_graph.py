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
