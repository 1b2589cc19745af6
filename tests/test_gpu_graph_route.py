"""Graph capture of a routed layer: route -> gather -> grouped forward ->
combine, plus the fp8 scale packing and forward, captured once and replayed
with new routings written in place on the device between replays (with
eager work and synchronisations in between).  Every replay must equal an
eager run on the same inputs bit for bit (all steps are deterministic), so
nothing about the routing is baked into the graph on the host."""
import numpy as np
import pytest

from moe_grouped_gemm_ragged_amd import binding as gg
from moe_grouped_gemm_ragged_amd import synth
from gpu_util import device, say

pytestmark = pytest.mark.gpu


def test_graph_routed_layer_follows_device_routing():
    import torch
    dev = device()
    tokens, topk, e, k, n = 600, 4, 24, 256, 264
    rng = np.random.default_rng(31)
    routings = [np.stack([rng.choice(e, topk, replace=False) for _ in range(tokens)]).astype(np.int32)
                for _ in range(4)]
    routings[2][:, 0] = 3                      # a skewed routing
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    x = torch.randn((tokens, k), generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn((e, k, n), generator=g, device=dev) * 0.05).to(torch.bfloat16)
    probs = torch.rand((tokens, topk), generator=g, device=dev)
    ids = torch.from_numpy(routings[0]).to(dev)
    cap = gg.route_rows_bound(tokens * topk, e, 16)
    ws = torch.empty(int(gg.load().gg_route_workspace_bytes(tokens * topk, e)), dtype=torch.uint8, device=dev)
    offs = torch.empty(e, dtype=torch.int32, device=dev)
    row_slot = torch.empty(cap, dtype=torch.int32, device=dev)
    slot_row = torch.empty(tokens * topk, dtype=torch.int32, device=dev)
    xg = torch.zeros((cap, k), dtype=torch.bfloat16, device=dev)
    y = torch.zeros((cap, n), dtype=torch.bfloat16, device=dev)
    out = torch.zeros((tokens, n), dtype=torch.bfloat16, device=dev)

    def layer(o):
        st = torch.cuda.current_stream(dev).cuda_stream
        assert gg.call_raw("gg_route", ids.data_ptr(), tokens * topk, e, 16, 1, offs.data_ptr(),
                           row_slot.data_ptr(), cap, slot_row.data_ptr(), ws.data_ptr(), st) == 0
        gg.gather_rows(x, row_slot, topk, offs, out=xg)
        gg.forward(xg, w, offs, out=y)
        gg.combine_rows(y, slot_row, topk, probs, out=o)

    say("graph routed layer: warm-up and capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer(out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer(out)
    torch.cuda.synchronize()
    eager = torch.empty_like(out)
    for rep, r in enumerate(routings[1:] + routings[:1]):
        ids.copy_(torch.from_numpy(r).to(dev))
        out.fill_(0)
        torch.cuda.synchronize()
        say("graph routed layer: replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        layer(eager)                            # eager run on the same routing
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"replay {rep} differs"


def test_graph_fp8_pack_and_forward():
    import torch
    dev = device()
    wl = synth.by_name("fp8_masked_down_small")
    t = synth.make_fp8_inputs(wl, dev)
    e = wl.num_groups
    xs = torch.empty(gg.fp8_scale_bytes(gg.GG_FP8_ACT_MASKED, wl.m, wl.k, e), dtype=torch.uint8, device=dev)
    ws = gg.fp8_pack_scales(gg.GG_FP8_WEIGHT, t["sw"], None, wl.n, wl.k, e)
    y = torch.zeros((e, wl.m, wl.n), dtype=torch.bfloat16, device=dev)
    mm = t["masked_m"]

    def step(o):
        gg.fp8_pack_scales(gg.GG_FP8_ACT_MASKED, t["sx"], mm, wl.m, wl.k, e, out=xs)
        gg.fp8_masked_forward(t["x8"], xs, t["w8"], ws, mm, out=o)

    say("graph fp8: warm-up and capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    eager = torch.empty_like(y)
    for rep in range(3):
        mm.copy_(torch.from_numpy(rng.integers(0, wl.m + 1, e).astype(np.int32)).to(dev))
        y.fill_(0)
        eager.fill_(0)
        torch.cuda.synchronize()
        say("graph fp8: replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        step(eager)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {rep} differs"
