"""GPU robustness: the edge cases of the ragged and masked grouped GEMM,
through the C ABI, against the fp64 oracle element by element.

* group sizes 0, 1, 7, 8, 9, 16, 127, 128, 129, 255, 256, 257 with empty
  experts first, in the middle and last, unused trailing rows, and K / N that
  are not multiples of the 256-wide tile (8-element tails);
* all experts empty, M = 0, a single expert (a dense GEMM), the maximum
  expert count;
* offsets that decrease or run past M, masked_m below 0 or above max_m
  (clamped: the oracle applies the same clamp);
* NaN in input rows no expert owns and in the weights of empty experts (never
  read, so it must not reach any output), NaN pre-filled in the outputs
  (overwritten where written, untouched elsewhere).
"""
import numpy as np
import pytest

import oracle
from moe_grouped_gemm_ragged_amd import binding as gg
from moe_grouped_gemm_ragged_amd import synth
from gpu_util import device, host, raw_bits, say, sentinel_bits, sentinel_tensor
from parity import Report, check

pytestmark = pytest.mark.gpu

EDGE_SIZES = [0, 1, 7, 8, 9, 16, 0, 127, 128, 129, 255, 256, 257, 0]


def _clamped_ends(offs, m):
    ends, prev = [], 0
    for o in offs:
        e = min(max(int(o), prev), m)
        ends.append(e)
        prev = e
    return np.array(ends, dtype=np.int64)


def _ragged(name, offs, m, k, n, seed):
    return synth.Workload(name, "ragged", len(offs), m, k, n, seed=seed,
                          offs=np.asarray(offs, dtype=np.int32))


def _run_all_passes(wl, t, out_dtype_fwd="bf16", nan_unused=False, nan_empty_w=False):
    """Runs fwd, dgrad and wgrad on sentinel-filled outputs and checks every
    element against the oracle (rows no expert owns must be untouched)."""
    import torch
    dev = t["x"].device
    ends = _clamped_ends(wl.offs, wl.m)
    used_total = int(ends[-1]) if len(ends) else 0
    sizes = np.diff(np.concatenate([[0], ends]))
    if nan_unused and used_total < wl.m:
        t["x"].view(torch.int16)[used_total:] = synth.BF16_QNAN
        t["dy"].view(torch.int16)[used_total:] = synth.BF16_QNAN
    if nan_empty_w:
        for g in np.nonzero(sizes == 0)[0]:
            t["w"].view(torch.int16)[int(g)] = synth.BF16_QNAN
    odt = {"bf16": torch.bfloat16, "f32": torch.float32}[out_dtype_fwd]
    y = sentinel_tensor((wl.m, wl.n), odt, dev)
    dx = sentinel_tensor((wl.m, wl.k), odt, dev)
    dw = sentinel_tensor((wl.num_groups, wl.k, wl.n), torch.float32, dev)
    say("robustness", wl.name, "fwd/dgrad/wgrad", out_dtype_fwd)
    gg.forward(t["x"], t["w"], t["offs"], out=y)
    gg.dgrad(t["dy"], t["w"], t["offs"], out=dx)
    gg.wgrad(t["x"], t["dy"], t["offs"], out=dw)
    torch.cuda.synchronize()
    hx, hw, hdy = (synth.bf16_bits(t[k]) for k in ("x", "w", "dy"))
    rep = Report()
    rf = oracle.forward(hx, hw, wl.offs)
    used = rf.status == 1
    assert int(used.sum()) == used_total
    yh = host(y)
    check(yh[used], rf.value[used], rf.sabs[used], wl.k, f"fwd {wl.name}", rep)
    assert np.all(raw_bits(yh[~used]) == sentinel_bits(odt)), "fwd wrote a row no expert owns"
    rd = oracle.dgrad(hdy, hw, wl.offs)
    dxh = host(dx)
    check(dxh[used], rd.value[used], rd.sabs[used], wl.n, f"dgrad {wl.name}", rep)
    assert np.all(raw_bits(dxh[~used]) == sentinel_bits(odt)), "dgrad wrote a row no expert owns"
    rw = oracle.wgrad(hx, hdy, wl.offs)
    dwh = host(dw).reshape(wl.num_groups * wl.k, wl.n)
    L = np.repeat(np.maximum(sizes, 1), wl.k)[:, None]
    check(dwh, rw.value, rw.sabs, L, f"wgrad {wl.name}", rep)
    empty = np.repeat(sizes == 0, wl.k)
    assert np.all(dwh[empty].view(np.uint32) == 0), "an empty expert's dW is not +0.0"
    assert np.all(np.isfinite(dwh)), "NaN reached dW"
    print(wl.name, rep)
    return y, dx, dw


@pytest.mark.parametrize("k,n", [(264, 520), (8, 8), (40, 264)])
def test_edge_group_sizes(k, n):
    dev = device()
    sizes = EDGE_SIZES
    wl = synth.custom_ragged(f"edge_{k}x{n}", sizes, k, n, seed=31 + k, m=int(sum(sizes)) + 40)
    t = synth.make_inputs(wl, dev)
    _run_all_passes(wl, t, nan_unused=True, nan_empty_w=True)


def test_edge_group_sizes_fp32_outputs():
    dev = device()
    wl = synth.custom_ragged("edge_f32", EDGE_SIZES, 136, 264, seed=41, m=int(sum(EDGE_SIZES)) + 3)
    t = synth.make_inputs(wl, dev)
    _run_all_passes(wl, t, out_dtype_fwd="f32", nan_unused=True)


def test_all_experts_empty():
    """No expert owns a row: forward and dgrad write nothing, wgrad writes
    +0.0 over all of dW."""
    dev = device()
    wl = _ragged("all_empty", [0, 0, 0, 0, 0], 64, 264, 136, seed=5)
    t = synth.make_inputs(wl, dev)
    _run_all_passes(wl, t, nan_unused=True)


def test_empty_first_and_last_only():
    dev = device()
    wl = synth.custom_ragged("empty_ends", [0, 300, 0, 513, 0], 72, 264, seed=6)
    t = synth.make_inputs(wl, dev)
    _run_all_passes(wl, t, nan_empty_w=True)


def test_single_expert_is_dense():
    dev = device()
    wl = _ragged("dense", [777], 777, 520, 264, seed=7)
    t = synth.make_inputs(wl, dev)
    _run_all_passes(wl, t)


def test_invalid_offsets_are_clamped():
    """Decreasing, negative and past-M offsets: the ends are clamped to a
    monotone sequence inside [0, M] (the oracle does the same); nothing
    outside the clamped rows is read or written."""
    dev = device()
    m = 600
    wl = _ragged("bad_offs", [-5, 100, 50, 300, 250, 10_000, 4], m, 136, 264, seed=8)
    assert list(_clamped_ends(wl.offs, m)) == [0, 100, 100, 300, 300, 600, 600]
    t = synth.make_inputs(wl, dev)
    _run_all_passes(wl, t)


def test_offsets_end_before_m():
    dev = device()
    wl = _ragged("short", [100, 230, 231], 1000, 264, 136, seed=9)
    t = synth.make_inputs(wl, dev)
    _run_all_passes(wl, t, nan_unused=True)


def test_max_expert_count():
    """GG_MAX_GROUPS experts, most of them empty or tiny."""
    import torch
    dev = device()
    E = 2048
    rng = np.random.default_rng(10)
    sizes = rng.choice([0, 0, 0, 1, 2, 3, 9], size=E)
    sizes[rng.integers(0, E, 3)] = 200
    wl = synth.custom_ragged("max_groups", sizes, 64, 72, seed=10)
    t = synth.make_inputs(wl, dev)
    assert t["w"].shape[0] == E
    _run_all_passes(wl, t)
    torch.cuda.empty_cache()


def test_zero_rows():
    """M = 0: forward and dgrad write nothing; wgrad writes +0.0 to dW."""
    import torch
    dev = device()
    E, k, n = 3, 64, 40
    x = torch.zeros((1, k), dtype=torch.bfloat16, device=dev)     # real buffers, m = 0
    dy = torch.zeros((1, n), dtype=torch.bfloat16, device=dev)
    w = torch.ones((E, k, n), dtype=torch.bfloat16, device=dev)
    offs = torch.tensor([0, 5, 7], dtype=torch.int32, device=dev)  # clamped to 0
    y = sentinel_tensor((1, n), torch.bfloat16, dev)
    dx = sentinel_tensor((1, k), torch.bfloat16, dev)
    dw = sentinel_tensor((E, k, n), torch.float32, dev)
    stream = torch.cuda.current_stream().cuda_stream
    say("zero rows")
    for name, a, b, c, dt in (("gg_forward", x, w, y, 0), ("gg_dgrad", dy, w, dx, 0),
                              ("gg_wgrad", x, dy, dw, 1)):
        rc = gg.call_raw(name, a.data_ptr(), b.data_ptr(), offs.data_ptr(), c.data_ptr(), dt,
                         0, k, n, E, stream)
        assert rc == 0, gg.last_error()
    torch.cuda.synchronize()
    assert np.all(host(y) == synth.OUT_SENTINEL_BF16)
    assert np.all(host(dx) == synth.OUT_SENTINEL_BF16)
    assert np.all(host(dw).view(np.uint32) == 0)


def test_nan_prefilled_outputs_are_overwritten():
    """beta = 0: outputs are never read, so NaN already in a written row
    must be replaced; rows no expert owns keep their NaN."""
    import torch
    dev = device()
    wl = synth.custom_ragged("nan_out", [33, 0, 260, 9], 136, 264, seed=12, m=330)
    t = synth.make_inputs(wl, dev)
    y = torch.full((wl.m, wl.n), float("nan"), dtype=torch.bfloat16, device=dev)
    dw = torch.full((wl.num_groups, wl.k, wl.n), float("nan"), dtype=torch.float32, device=dev)
    say("nan-prefilled outputs")
    gg.forward(t["x"], t["w"], t["offs"], out=y)
    gg.wgrad(t["x"], t["dy"], t["offs"], out=dw)
    torch.cuda.synchronize()
    used = int(wl.offs[-1])
    yh = host(y)
    hx, hw, hdy = (synth.bf16_bits(t[k]) for k in ("x", "w", "dy"))
    rf = oracle.forward(hx, hw, wl.offs)
    check(yh[:used], rf.value[:used], rf.sabs[:used], wl.k, "fwd over NaN")
    tail = synth.bf16_bits(y[used:])
    assert np.all((tail & 0x7F80) == 0x7F80) and np.all((tail & 0x7F) != 0), "an unowned row lost its NaN"
    dwh = host(dw)
    assert np.all(np.isfinite(dwh)), "dW kept a NaN"
    rw = oracle.wgrad(hx, hdy, wl.offs)
    L = np.repeat(np.maximum(wl.group_sizes(), 1), wl.k)[:, None]
    check(dwh.reshape(-1, wl.n), rw.value, rw.sabs, L, "wgrad over NaN")


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_masked_extremes(out):
    """masked_m of 0, 8, max_m, above max_m and negative (clamped into
    [0, max_m]); inactive X rows hold NaN and inactive Y rows a sentinel."""
    import torch
    dev = device()
    max_m, k, n = 256, 264, 136
    mm = np.array([0, 8, 256, 300, -3, 100, 1, 255, 129], dtype=np.int32)
    wl = synth.custom_masked("masked_edge", mm, max_m, k, n, seed=13)
    t = synth.make_inputs(wl, dev, need=("x", "w"))
    odt = {"bf16": torch.bfloat16, "f32": torch.float32}[out]
    y = sentinel_tensor((wl.num_groups, max_m, n), odt, dev)
    say("masked extremes", out)
    gg.masked_forward(t["x"], t["w"], t["masked_m"], out=y)
    torch.cuda.synchronize()
    ref = oracle.masked_forward(synth.bf16_bits(t["x"]), synth.bf16_bits(t["w"]), mm)
    act = ref.status == 1
    active_rows = np.clip(mm, 0, max_m)
    assert int(act.sum()) == int(active_rows.sum())
    yh = host(y).reshape(wl.num_groups * max_m, n)
    rep = Report()
    check(yh[act], ref.value[act], ref.sabs[act], k, "masked extremes", rep)
    assert np.all(raw_bits(yh[~act]) == sentinel_bits(odt)), "an inactive row was written"
    print(out, rep)


@pytest.mark.parametrize("e,k,n", [(512, 64, 72), (513, 64, 72), (100, 296, 520)])
def test_wgrad_expert_order_boundary(e, k, n):
    """wgrad takes its experts longest first (and alternates the direction of
    its rounds) up to 512 experts, in index order above: 512 and 513 experts
    of one tile each (two rounds of the 256-workgroup grid), and 100 experts
    of 6 tiles each (2.3 rounds); sizes skewed (many empty or tiny, a few
    large) so that the order differs from the index order.  Every pass is
    checked against the oracle on every element."""
    import torch
    dev = device()
    rng = np.random.default_rng(e + k)
    sizes = rng.choice([0, 0, 1, 5, 17, 40], size=e)
    big = rng.choice(e, size=max(2, e // 40), replace=False)
    sizes[big] = rng.integers(200, 700, size=len(big))
    wl = synth.custom_ragged(f"wgrad_order_{e}", sizes, k, n, seed=e + 3)
    t = synth.make_inputs(wl, dev)
    _run_all_passes(wl, t)
    torch.cuda.empty_cache()
