"""GPU-only invariants of the grouped GEMM kernels (they pin properties the
oracle comparison alone would not):

* repeat calls are bit-identical (fixed tile decomposition, no atomics);
* forward(2 X) == 2 forward(X) and dgrad(2 dY) == 2 dgrad(dY) bit for bit
  (scaling by two is exact and the rounding commutes with it);
* permuting rows inside each expert permutes the forward and dgrad outputs
  bit for bit (each output element's reduction does not depend on where its
  row sits in a tile);
* the masked forward of a compacted layout equals the ragged forward on the
  same rows (two layouts, one operation).
"""
import numpy as np
import pytest

from moe_grouped_gemm_ragged_amd import binding as gg
from moe_grouped_gemm_ragged_amd import synth
from gpu_util import device, say

pytestmark = pytest.mark.gpu


def _wl():
    return synth.custom_ragged("inv", [0, 129, 7, 300, 0, 256, 41], 264, 520, seed=55, m=760)


def test_repeat_calls_bit_identical():
    import torch
    dev = device()
    wl = _wl()
    t = synth.make_inputs(wl, dev)
    outs = []
    say("determinism")
    for _ in range(3):
        y = torch.zeros((wl.m, wl.n), dtype=torch.bfloat16, device=dev)
        dx = torch.zeros((wl.m, wl.k), dtype=torch.bfloat16, device=dev)
        dw = torch.zeros((wl.num_groups, wl.k, wl.n), dtype=torch.float32, device=dev)
        gg.forward(t["x"], t["w"], t["offs"], out=y)
        gg.dgrad(t["dy"], t["w"], t["offs"], out=dx)
        gg.wgrad(t["x"], t["dy"], t["offs"], out=dw)
        outs.append((y, dx, dw))
    torch.cuda.synchronize()
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_scaling_by_two_is_exact():
    import torch
    dev = device()
    wl = _wl()
    t = synth.make_inputs(wl, dev)
    used = int(wl.offs[-1])
    say("scale by two")
    y1 = gg.forward(t["x"], t["w"], t["offs"])
    y2 = gg.forward(t["x"] * 2, t["w"], t["offs"])
    d1 = gg.dgrad(t["dy"], t["w"], t["offs"])
    d2 = gg.dgrad(t["dy"] * 2, t["w"], t["offs"])
    w1 = gg.wgrad(t["x"], t["dy"], t["offs"])
    w2 = gg.wgrad(t["x"] * 2, t["dy"], t["offs"])
    torch.cuda.synchronize()
    assert torch.equal(y2[:used], y1[:used] * 2)
    assert torch.equal(d2[:used], d1[:used] * 2)
    assert torch.equal(w2, w1 * 2)


def test_row_permutation_within_experts():
    import torch
    dev = device()
    wl = _wl()
    t = synth.make_inputs(wl, dev)
    rng = np.random.default_rng(3)
    perm = np.arange(wl.m)
    start = 0
    for end in wl.offs:
        perm[start:end] = start + rng.permutation(end - start)
        start = end
    p = torch.from_numpy(perm).to(dev)
    used = int(wl.offs[-1])
    say("row permutation")
    y = gg.forward(t["x"], t["w"], t["offs"])
    yp = gg.forward(t["x"][p].contiguous(), t["w"], t["offs"])
    dx = gg.dgrad(t["dy"], t["w"], t["offs"])
    dxp = gg.dgrad(t["dy"][p].contiguous(), t["w"], t["offs"])
    torch.cuda.synchronize()
    assert torch.equal(yp[:used], y[p][:used])
    assert torch.equal(dxp[:used], dx[p][:used])


def test_masked_equals_ragged_on_compacted_rows():
    import torch
    dev = device()
    max_m, k, n = 256, 264, 136
    mm = np.array([5, 0, 256, 130, 8, 77], dtype=np.int32)
    wm = synth.custom_masked("mvr", mm, max_m, k, n, seed=66)
    t = synth.make_inputs(wm, dev, need=("x", "w"))
    rows = torch.cat([t["x"][e, :int(mm[e])] for e in range(len(mm))]).contiguous()
    offs = torch.from_numpy(np.cumsum(mm).astype(np.int32)).to(dev)
    say("masked vs ragged")
    ym = gg.masked_forward(t["x"], t["w"], t["masked_m"])
    yr = gg.forward(rows, t["w"], offs)
    torch.cuda.synchronize()
    got = torch.cat([ym[e, :int(mm[e])] for e in range(len(mm))])
    assert torch.equal(got, yr)


def test_concurrent_streams_match_serial():
    """The library keeps no device state between calls (no workspace, no
    counters): the four passes launched together on four streams, each
    kernel persistent over every CU, give the same bits as one after another
    on one stream, and leave the rows they must not write untouched."""
    import torch
    dev = device()
    wl = _wl()
    t = synth.make_inputs(wl, dev)
    mwl = synth.masked_down("small")
    mt = synth.make_inputs(mwl, dev, need=("x", "w"))
    used = int(t["offs"][-1])
    mm = mt["masked_m"].to(torch.int64).cpu()
    active = (torch.arange(mwl.m)[None, :] < mm[:, None]).to(dev)     # [E, max_m]
    sentinel = -63             # 0xFFC1 (bf16) or 0xFFFFFFC1 (fp32): a NaN no pass writes
    say("concurrent streams")

    def bits(x):
        return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)

    def prefilled(shape, dtype):
        o = torch.empty(shape, dtype=dtype, device=dev)
        bits(o).fill_(sentinel)
        return o

    y0 = prefilled((wl.m, wl.n), torch.bfloat16)
    dx0 = prefilled((wl.m, wl.k), torch.bfloat16)
    dw0 = prefilled((wl.num_groups, wl.k, wl.n), torch.float32)
    ym0 = prefilled((mwl.num_groups, mwl.m, mwl.n), torch.bfloat16)
    gg.forward(t["x"], t["w"], t["offs"], out=y0)
    gg.dgrad(t["dy"], t["w"], t["offs"], out=dx0)
    gg.wgrad(t["x"], t["dy"], t["offs"], out=dw0)
    gg.masked_forward(mt["x"], mt["w"], mt["masked_m"], out=ym0)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev) for _ in range(4)]
    main = torch.cuda.current_stream(dev)
    calls = (lambda o: gg.forward(t["x"], t["w"], t["offs"], out=o),
             lambda o: gg.dgrad(t["dy"], t["w"], t["offs"], out=o),
             lambda o: gg.wgrad(t["x"], t["dy"], t["offs"], out=o),
             lambda o: gg.masked_forward(mt["x"], mt["w"], mt["masked_m"], out=o))
    for rep in range(3):
        outs = [prefilled(r.shape, r.dtype) for r in (y0, dx0, dw0, ym0)]
        for s in streams:
            s.wait_stream(main)
        for s, o, call in zip(streams, outs, calls):
            with torch.cuda.stream(s):
                call(o)
        for s in streams:
            main.wait_stream(s)
        torch.cuda.synchronize()
        for name, got, want in zip(("forward", "dgrad", "wgrad", "masked forward"), outs, (y0, dx0, dw0, ym0)):
            assert torch.equal(bits(got), bits(want)), f"{name} differs on concurrent streams (repeat {rep})"
    # the serial outputs themselves: rows past the last offset and inactive
    # masked rows kept the sentinel, every written element did not
    assert bool((bits(y0[used:]) == sentinel).all()) and bool((bits(dx0[used:]) == sentinel).all())
    assert not bool((bits(y0[:used]) == sentinel).any()) and not bool((bits(dw0) == sentinel).any())
    assert bool((bits(ym0)[~active] == sentinel).all()) and not bool((bits(ym0)[active] == sentinel).any())
