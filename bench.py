#!/usr/bin/env python3
"""Benchmark of the bf16 grouped GEMM on one MI355X.

One step = the three passes of the grouped GEMM (forward, dgrad, wgrad) over
the GLM-up workload: 32 experts, 262144 rows, K = 6144, N = 4096, group sizes
Dirichlet(1) proportions rounded to multiples of 128 (TileOPs issue #1566,
"Summary", gives the shape).  Inputs are seeded synthetic bf16 data already
resident in HBM; outputs are preallocated caller buffers (bf16 Y and dX,
fp32 dW).  The line printed is whole-job TFLOP/s over the timed steps
(3 x 2 x rows x K x N FLOP per step).

Also reported: per-pass times from HIP events on the launch stream, the
roofline object for the dominant kernel, the masked down-projection workload
and the other shapes as context, and the fp64 CPU oracle timed on a bounded
sample of the same workload (cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Profiling helpers (each prints one JSON line of its own, not the bench line):
  --profile-pass {fwd,dgrad,wgrad}  run only that pass of the workload
  --profile-workload NAME           ... of this workload instead (glm_up,
                                    qwen3_gateup or dsv3)
  --copy-calibration                run a plain device-to-device copy of known
                                    size, to scale the FETCH_SIZE / WRITE_SIZE
                                    counters into bytes
  --tile-cost                       time the forward on uniform-expert shapes at
                                    Qwen3's N: full- against half-height tiles,
                                    and a reduction-length sweep that separates a
                                    tile's fixed cost from its per-stage time
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 bf16 FLOP/clk/CU (dense)
PEAK_FP8_TFLOPS = 5033.2       # the same with e4m3 operands (8192 FLOP/clk/CU, dense)
PEAK_HBM_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "moe_grouped_gemm_ragged_amd", "csrc", "gg_kernels.hip")

# Counter readings of the kernel, from rocprofv3 --pmc runs of
# `bench.py --profile-pass P --profile-workload W` (the summaries under
# profiles/ give the commands and every reading):
#   traffic: HBM-side bytes per launch, FETCH_SIZE and WRITE_SIZE each divided
#     by the factor the same counter reads for `bench.py --copy-calibration`;
#   clock_GHz: sustained shader clock, GRBM_GUI_ACTIVE / 8 XCDs / kernel time;
#   mfma_busy: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles per XCD).
# Last dispatch of each run.  Valid only for the kernel source they were
# taken on (sha256 below); for any other source these fields are null.
MEASURED = {
    "kernel_sha256": "fbc9d9e2fa630706c99cd2325ef5af9eecdadec198cf289f466880c1d3c842f2",
    "glm_up": {"fwd": {"traffic": 23623406989, "clock_GHz": 1.564, "mfma_busy": 0.791},
              "dgrad": {"traffic": 28929209119, "clock_GHz": 1.582, "mfma_busy": 0.757},
              "wgrad": {"traffic": 23134283872, "clock_GHz": 1.576, "mfma_busy": 0.801}},
    "qwen3_gateup": {"fwd": {"traffic": 1853467875, "clock_GHz": 1.954, "mfma_busy": 0.491},
                    "dgrad": {"traffic": 1901057487, "clock_GHz": 1.772, "mfma_busy": 0.461},
                    "wgrad": {"traffic": 2375981198, "clock_GHz": 1.915, "mfma_busy": 0.304}},
    "dsv3": {"fwd": {"traffic": 8458537885},
            "dgrad": {"traffic": 9091197942},
            "wgrad": {"traffic": 16687648838}},
}
NOMINAL_CLOCK_GHZ = 2.4


def measured(workload, pass_, key):
    """A counter reading of MEASURED for this kernel source, else None."""
    if MEASURED["kernel_sha256"] != kernel_sha256():
        return None
    return MEASURED.get(workload, {}).get(pass_, {}).get(key)


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def kernel_sha256():
    """sha256 of the kernel source's code: comments and blank lines removed,
    so that a comment edit does not invalidate counter measurements."""
    with open(KERNEL_SRC) as f:
        src = f.read()
    src = re.sub(r"//[^\n]*", "", src)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    code = "\n".join(line.strip() for line in src.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def time_passes(fns, steps, warmup, torch):
    """Run the list of (name, fn) ``warmup`` times, then ``steps`` times with
    HIP events around every launch.  Returns (total seconds, {name: [ms]})."""
    for _ in range(warmup):
        for _, f in fns:
            f()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = {name: [] for name, _ in fns}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for name, f in fns:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f()
            b.record(stream)
            evs[name].append((a, b))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = {name: [a.elapsed_time(b) for a, b in v] for name, v in evs.items()}
    return t1 - t0, ms


def device_info(torch):
    """CU count and peak engine clock as the HIP runtime reports them, and the
    dense bf16 MFMA peak they imply (CUs x clock x 4096 FLOP/clk/CU).  The
    roofline keeps the published 2516.6 TFLOP/s; this is the cross-check."""
    import ctypes
    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count,
            "hbm_GiB": round(props.total_memory / 2**30, 1)}
    try:
        path = next(line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64.so" in line)
        hip = ctypes.CDLL(path)
        khz = ctypes.c_int(0)
        # hipDeviceAttributeClockRate (5): peak engine clock in kHz
        if hip.hipDeviceGetAttribute(ctypes.byref(khz), ctypes.c_int(5), ctypes.c_int(0)) == 0 and khz.value > 0:
            info["max_sclk_MHz"] = khz.value // 1000
            info["bf16_peak_from_device_TFLOP/s"] = round(props.multi_processor_count * khz.value * 1e3 * 4096 / 1e12, 1)
    except (StopIteration, OSError, AttributeError):
        pass
    return info


def algorithmic_bytes(wl, pass_):
    """Bytes the pass must move at minimum: active rows of its inputs and
    outputs and the weights of experts with rows (wgrad: all of fp32 dW)."""
    import numpy as np
    sizes = wl.group_sizes()
    rows = int(sizes.sum())
    live = int((sizes > 0).sum())
    k, n = wl.k, wl.n
    if pass_ == "fwd":
        return 2 * rows * k + 2 * live * k * n + 2 * rows * n
    if pass_ == "dgrad":
        return 2 * rows * n + 2 * live * k * n + 2 * rows * k
    if pass_ == "wgrad":
        return 2 * rows * k + 2 * rows * n + 4 * wl.num_groups * k * n
    raise ValueError(pass_)


def cpu_baseline(wl, t, synth, budget_s=15.0):
    """The fp64 oracle on a bounded sample of the same workload: rows of the
    forward and dgrad, (expert, k) rows of the wgrad, each sized from a short
    calibration run to take about budget_s / 3 seconds."""
    import numpy as np
    import oracle
    hb = {k: synth.bf16_bits(t[k]) for k in ("x", "w", "dy")}
    rng = np.random.default_rng(2024)
    total = wl.active_rows()
    sizes = wl.group_sizes()
    flops = 0.0
    secs = 0.0
    parts = []
    per_pass = {}

    def timed(fn, *args, **kw):
        t0 = time.perf_counter()
        fn(*args, **kw)
        return time.perf_counter() - t0

    # forward / dgrad: calibrate on 64 rows, then size the sample
    for name, fn, a, per_row in (("forward", oracle.forward, (hb["x"], hb["w"], wl.offs), 2.0 * wl.k * wl.n),
                                 ("dgrad", oracle.dgrad, (hb["dy"], hb["w"], wl.offs), 2.0 * wl.k * wl.n)):
        cal = rng.integers(0, total, 64)
        dt = timed(fn, *a, rows=cal)
        rate = 64 * per_row / max(dt, 1e-6)
        nrows = int(min(max(64, rate * budget_s / 3 / per_row), total))
        rows = rng.integers(0, total, nrows)
        dt = timed(fn, *a, rows=rows)
        flops += nrows * per_row
        secs += dt
        parts.append(f"{name}: {nrows} random rows")
        per_pass[name] = {"GFLOP": round(nrows * per_row / 1e9, 2), "seconds": round(dt, 2),
                          "GFLOP/s": round(nrows * per_row / dt / 1e9, 1)}
    # wgrad: (expert, k) rows of dW, expert chosen with probability ~ rows
    live = np.nonzero(sizes > 0)[0]
    p = sizes[live] / sizes[live].sum()
    mean_cost = 2.0 * float((sizes[live] * p).sum()) * wl.n
    cal_pairs = np.stack([rng.choice(live, 8, p=p), rng.integers(0, wl.k, 8)], axis=1)
    dt = timed(oracle.wgrad, hb["x"], hb["dy"], wl.offs, pairs=cal_pairs)
    cost = 2.0 * float(sizes[cal_pairs[:, 0]].sum()) * wl.n
    rate = cost / max(dt, 1e-6)
    npairs = int(max(8, rate * budget_s / 3 / mean_cost))
    pairs = np.stack([rng.choice(live, npairs, p=p), rng.integers(0, wl.k, npairs)], axis=1)
    dt = timed(oracle.wgrad, hb["x"], hb["dy"], wl.offs, pairs=pairs)
    wf = 2.0 * float(sizes[pairs[:, 0]].sum()) * wl.n
    flops += wf
    secs += dt
    parts.append(f"wgrad: {npairs} (expert, k) rows of dW")
    per_pass["wgrad"] = {"GFLOP": round(wf / 1e9, 2), "seconds": round(dt, 2), "GFLOP/s": round(wf / dt / 1e9, 1)}
    return {
        "value": flops / secs / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{wl.name}, {'; '.join(parts)}; {flops / 1e9:.1f} GFLOP in {secs:.1f} s",
        "per_pass": per_pass,
    }


def tile_cost(gg, synth, torch, dev, n=1536, experts=256, cus=256):
    """Forward time per output tile on uniform experts (every expert the same
    size, 256-column tiles at n = 1536): 256-row experts (one full-height tile
    each), 192 rows (one full-height tile, partly empty), 128 rows (one
    half-height tile), all at k = 2048; and 256-row experts at k = 512 ..
    4096, whose least-squares line in the stage count (k / 32) gives a tile's
    fixed cost (intercept) and its time per stage (slope), for bf16 output
    (stored through LDS) and fp32 output (stored straight from the
    accumulators, overlapped with the next tile's first loads); and the same
    split for wgrad on 64 uniform experts of 128 .. 1024 rows (fp32 dW).
    Times are per workgroup: launch time x CUs / tiles."""
    import numpy as np
    col_tiles = (n + 255) // 256
    out = {"n": n, "experts": experts, "col_tiles": col_tiles, "shapes": []}

    def run(rows, k, out_dtype=torch.bfloat16):
        wl = synth.custom_ragged(f"uniform_{rows}x{k}", [rows] * experts, k=k, n=n, seed=77)
        t = synth.make_inputs(wl, dev, need=("x", "w"))
        y = torch.empty((wl.m, wl.n), dtype=out_dtype, device=dev)
        _, ms = time_passes([("fwd", lambda: gg.forward(t["x"], t["w"], t["offs"], out=y))], 20, 3, torch)
        med = sorted(ms["fwd"])[len(ms["fwd"]) // 2]
        tiles = experts * col_tiles
        e = {"rows": rows, "k": k, "out": str(out_dtype).replace("torch.", ""), "stages": k // 32,
             "ms": round(med, 4), "tiles_per_cu": tiles / cus,
             "us_per_tile": round(med * 1e3 * cus / tiles, 2),
             "TFLOP/s": round(wl.flops() / (med * 1e-3) / 1e12, 1)}
        out["shapes"].append(e)
        del t, y
        return e
    full = run(256, 2048)
    run(192, 2048)
    half = run(128, 2048)
    out["half_over_full_tile_time"] = round(half["us_per_tile"] / full["us_per_tile"], 3)
    for dt, sweep in ((torch.bfloat16, [full] + [run(256, k) for k in (512, 1024, 4096)]),
                      (torch.float32, [run(256, k, torch.float32) for k in (512, 1024, 2048, 4096)])):
        st = np.array([e["stages"] for e in sweep], dtype=float)
        us = np.array([e["us_per_tile"] for e in sweep])
        slope, icpt = np.polyfit(st, us, 1)
        tag = str(dt).replace("torch.", "")
        out[f"fit_{tag}_us_per_stage"] = round(float(slope), 4)
        out[f"fit_{tag}_fixed_us_per_tile"] = round(float(icpt), 2)
    # wgrad on 64 uniform experts of 128 .. 1024 rows at k = 2048, n = 1536
    # (48 dW tiles of 256 KB fp32 per expert; a stage is 32 of its rows)
    wg, k_w, e_w = [], 2048, 64
    tiles_w = e_w * (k_w // 256) * col_tiles
    for rows in (128, 256, 512, 1024):
        wl = synth.custom_ragged(f"uniform_wgrad_{rows}", [rows] * e_w, k=k_w, n=n, seed=78)
        t = synth.make_inputs(wl, dev, need=("x", "dy"))
        dw = torch.empty((e_w, k_w, n), dtype=torch.float32, device=dev)
        _, ms = time_passes([("w", lambda: gg.wgrad(t["x"], t["dy"], t["offs"], out=dw))], 20, 3, torch)
        med = sorted(ms["w"])[len(ms["w"]) // 2]
        wg.append({"rows": rows, "stages": rows // 32, "ms": round(med, 4),
                   "us_per_tile": round(med * 1e3 * cus / tiles_w, 2),
                   "algorithmic_GB/s": round(algorithmic_bytes(wl, "wgrad") / (med * 1e-3) / 1e9, 1)})
        del t, dw
    st = np.array([e["stages"] for e in wg], dtype=float)
    us = np.array([e["us_per_tile"] for e in wg])
    slope, icpt = np.polyfit(st, us, 1)
    out["wgrad_shapes"] = wg
    out["fit_wgrad_us_per_stage"] = round(float(slope), 4)
    out["fit_wgrad_fixed_us_per_tile"] = round(float(icpt), 2)
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the other workloads reported as context")
    ap.add_argument("--profile-pass", choices=("fwd", "dgrad", "wgrad"),
                    help="run only this pass (for counter collection) and exit")
    ap.add_argument("--profile-workload", default="glm_up",
                    choices=("glm_up", "qwen3_gateup", "dsv3"),
                    help="the workload --profile-pass runs (default glm_up, the bench workload)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain copy of known size (counter calibration) and exit")
    ap.add_argument("--tile-cost", action="store_true",
                    help="time full- against half-height tiles and a reduction sweep, then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(there is no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch

    from moe_grouped_gemm_ragged_amd import binding as gg
    from moe_grouped_gemm_ragged_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    gg.load()

    if args.copy_calibration:
        nbytes = 1 << 30
        src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        _, msc = time_passes([("copy", lambda: dst.copy_(src))], args.steps, args.warmup, torch)
        print(json.dumps({"copy_calibration": {"bytes_read": nbytes, "bytes_written": nbytes,
                                               "launches": args.warmup + args.steps,
                                               "ms": round(sum(msc["copy"]) / len(msc["copy"]), 4)}}),
              flush=True)
        return

    if args.tile_cost:
        print(json.dumps({"tile_cost": tile_cost(gg, synth, torch, dev)}), flush=True)
        return

    wl = synth.by_name(args.profile_workload) if args.profile_pass else synth.glm_up()
    log("generating", wl.name)
    t = synth.make_inputs(wl, dev)
    y = torch.empty((wl.m, wl.n), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((wl.m, wl.k), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((wl.num_groups, wl.k, wl.n), dtype=torch.float32, device=dev)
    fns = [
        ("fwd", lambda: gg.forward(t["x"], t["w"], t["offs"], out=y)),
        ("dgrad", lambda: gg.dgrad(t["dy"], t["w"], t["offs"], out=dx)),
        ("wgrad", lambda: gg.wgrad(t["x"], t["dy"], t["offs"], out=dw)),
    ]
    if args.profile_pass:
        one = [f for f in fns if f[0] == args.profile_pass]
        _, msp = time_passes(one, args.steps, args.warmup, torch)
        v = msp[args.profile_pass]
        print(json.dumps({"profile_pass": args.profile_pass, "workload": wl.name,
                          "launches": args.warmup + args.steps,
                          "ms": round(sum(v) / len(v), 4),
                          "TFLOP/s": round(wl.flops() / (sum(v) / len(v) * 1e-3) / 1e12, 2)}), flush=True)
        return
    log("timing", args.steps, "steps after", args.warmup, "warmup steps")
    secs, ms = time_passes(fns, args.steps, args.warmup, torch)
    flop_pass = wl.flops()
    flop_step = 3 * flop_pass
    value = flop_step * args.steps / secs / 1e12

    per_pass = {}
    for name in ("fwd", "dgrad", "wgrad"):
        avg = sum(ms[name]) / len(ms[name])
        tf = flop_pass / (avg * 1e-3) / 1e12
        per_pass[name] = {"ms": round(avg, 4), "TFLOP/s": round(tf, 2),
                          "frac_of_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                          "algorithmic_GB/s": round(algorithmic_bytes(wl, name) / (avg * 1e-3) / 1e9, 1)}
        # frac_of_mfma_peak ~ (clock / 2.4 GHz) x MFMA busy, from the counters
        clk, busy = measured(wl.name, name, "clock_GHz"), measured(wl.name, name, "mfma_busy")
        per_pass[name]["sustained_clock_GHz"] = clk
        per_pass[name]["mfma_busy"] = busy
        per_pass[name]["clock_x_busy"] = (round(clk / NOMINAL_CLOCK_GHZ * busy, 4)
                                          if clk is not None and busy is not None else None)
    dom = max(per_pass, key=lambda k: per_pass[k]["ms"])
    kernel_names = {"fwd": "grouped_gemm_kernel<0,false,false,false>", "dgrad": "grouped_gemm_kernel<1,false,false,false>",
                    "wgrad": "grouped_gemm_kernel<2,true,false,false>"}
    # wgrad accumulating into the fp32 main-grad (beta = 1), same workload
    _, msa = time_passes([("wgrad_acc", lambda: gg.wgrad(t["x"], t["dy"], t["offs"], out=dw, beta=1.0))],
                         3, 1, torch)
    acc_ms = sorted(msa["wgrad_acc"])[1]
    per_pass["wgrad_accumulate"] = {"ms": round(acc_ms, 4),
                                    "TFLOP/s": round(flop_pass / (acc_ms * 1e-3) / 1e12, 2),
                                    "note": "dW += X^T dY into fp32 (gg_wgrad_ex, beta = 1); not in the step"}

    traffic = measured(wl.name, dom, "traffic")
    roofline = {
        "bound": "mfma",
        "kernel": f"{kernel_names[dom]} ({dom})",
        "achieved": per_pass[dom]["TFLOP/s"],
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(per_pass[dom]["TFLOP/s"] / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic,
        "traffic_unit": "bytes per launch (HBM, counter-measured)",
        "algorithmic_bytes": algorithmic_bytes(wl, dom),
    }

    context = {}
    if not args.no_context:
        for name in ("qwen3_gateup", "dsv3"):
            w2 = synth.by_name(name)
            t2 = synth.make_inputs(w2, dev)
            y2 = torch.empty((w2.m, w2.n), dtype=torch.bfloat16, device=dev)
            dx2 = torch.empty((w2.m, w2.k), dtype=torch.bfloat16, device=dev)
            dw2 = torch.empty((w2.num_groups, w2.k, w2.n), dtype=torch.float32, device=dev)
            f2 = [("fwd", lambda: gg.forward(t2["x"], t2["w"], t2["offs"], out=y2)),
                  ("dgrad", lambda: gg.dgrad(t2["dy"], t2["w"], t2["offs"], out=dx2)),
                  ("wgrad", lambda: gg.wgrad(t2["x"], t2["dy"], t2["offs"], out=dw2))]
            _, ms2 = time_passes(f2, 10, 3, torch)
            entry = {}
            for p, v in ms2.items():
                avg = sorted(v)[len(v) // 2]
                gbs = algorithmic_bytes(w2, p) / (avg * 1e-3) / 1e9
                tf2 = w2.flops() / (avg * 1e-3) / 1e12
                entry[p] = {"ms": round(avg, 4), "TFLOP/s": round(tf2, 2),
                            "frac_of_mfma_peak": round(tf2 / PEAK_BF16_TFLOPS, 4),
                            "algorithmic_GB/s": round(gbs, 1),
                            "frac_of_hbm": round(gbs / PEAK_HBM_GBS, 4),
                            "traffic": measured(name, p, "traffic"),
                            "sustained_clock_GHz": measured(name, p, "clock_GHz"),
                            "mfma_busy": measured(name, p, "mfma_busy")}
            context[name] = entry
            del t2, y2, dx2, dw2
        # masked down-projection: forward and backward.  Its weights (201 MB)
        # fit in the 256 MB MALL, so they rotate over three copies and every
        # call streams them from HBM as a real layer would.
        wm = synth.masked_down()
        tm = synth.make_inputs(wm, dev, need=("x", "w", "dy"))
        wcopies = [tm["w"]] + [tm["w"].clone() for _ in range(2)]
        ym = torch.empty((wm.num_groups, wm.m, wm.n), dtype=torch.bfloat16, device=dev)
        dxm = torch.empty((wm.num_groups, wm.m, wm.k), dtype=torch.bfloat16, device=dev)
        dwm = [torch.empty((wm.num_groups, wm.k, wm.n), dtype=torch.float32, device=dev) for _ in range(3)]
        rot = {"i": 0}

        def nxt():
            rot["i"] = (rot["i"] + 1) % 3
            return rot["i"]
        live = int((wm.group_sizes() > 0).sum())
        act_rows = wm.active_rows()
        mb = {"masked_fwd": 2 * act_rows * (wm.k + wm.n) + 2 * live * wm.k * wm.n,
              "masked_dgrad": 2 * act_rows * (wm.k + wm.n) + 2 * live * wm.k * wm.n,
              "masked_wgrad": 2 * act_rows * (wm.k + wm.n) + 4 * wm.num_groups * wm.k * wm.n}
        fm = [("masked_fwd", lambda: gg.masked_forward(tm["x"], wcopies[nxt()], tm["masked_m"], out=ym)),
              ("masked_dgrad", lambda: gg.masked_dgrad(tm["dy"], wcopies[nxt()], tm["masked_m"], out=dxm)),
              ("masked_wgrad", lambda: gg.masked_wgrad(tm["x"], tm["dy"], tm["masked_m"], out=dwm[nxt()]))]
        _, msm = time_passes(fm, 30, 5, torch)
        entry = {"weights": "rotated over 3 copies (HBM-resident per call)"}
        for name, v in msm.items():
            avg = sorted(v)[len(v) // 2]
            gbs = mb[name] / (avg * 1e-3) / 1e9
            entry[name] = {"ms": round(avg, 4), "TFLOP/s": round(wm.flops() / (avg * 1e-3) / 1e12, 2),
                           "algorithmic_GB/s": round(gbs, 1), "frac_of_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        context["masked_down"] = entry
        del tm, wcopies, ym, dxm, dwm
        torch.cuda.empty_cache()

        # Qwen3 gate/up with the SiLU-mul activation fused into the epilogue,
        # against the plain forward followed by torch's SiLU-mul
        wq = synth.qwen3_gateup()
        tq = synth.make_inputs(wq, dev, need=("x", "w"))
        inter = wq.n // 2
        aq = torch.empty((wq.m, inter), dtype=torch.bfloat16, device=dev)
        hq = torch.empty((wq.m, wq.n), dtype=torch.bfloat16, device=dev)

        def unfused():
            gg.forward(tq["x"], tq["w"], tq["offs"], out=hq)
            torch.mul(torch.nn.functional.silu(hq[:, :inter]), hq[:, inter:], out=aq)
        _, msq = time_passes([("fused", lambda: gg.forward_silu_mul(tq["x"], tq["w"], tq["offs"], out=aq)),
                              ("unfused", unfused)], 10, 3, torch)
        fq = {k: sorted(v)[len(v) // 2] for k, v in msq.items()}
        context["qwen3_gateup_silu_mul"] = {
            "fused_ms": round(fq["fused"], 4),
            "fused_TFLOP/s": round(wq.flops() / (fq["fused"] * 1e-3) / 1e12, 2),
            "unfused_ms": round(fq["unfused"], 4),
            "unfused": "gg_forward to a bf16 [M, 2I] buffer, then torch silu(G) * U"}
        del tq, aq, hq
        torch.cuda.empty_cache()

        # The grouped layout's production and its consumers on a Qwen3
        # gate/up layer (8192 tokens, top-8 of 128 experts, min_alignment_m
        # 16 with empty experts padded): routing, the row gather, the
        # forward on the padded layout, the weighted combine; and the
        # forward with the grouped bias scaled per token against the plain
        # forward; and the bias term's backward (dbias and the per-token
        # factor's gradient) with the forward output standing in for dY.
        w4 = synth.qwen3_gateup()
        tokens4, topk4 = w4.m // 8, 8
        g4 = torch.Generator(device=dev)
        g4.manual_seed(404)
        scores = torch.randn((tokens4, w4.num_groups), generator=g4, device=dev)
        probs4, ids4 = torch.topk(torch.softmax(scores, -1), topk4, dim=-1)
        ids4 = ids4.to(torch.int32).contiguous()
        probs4 = probs4.float().contiguous()
        x4 = torch.randn((tokens4, w4.k), generator=g4, device=dev).to(torch.bfloat16)
        wt4 = (torch.randn((w4.num_groups, w4.k, w4.n), generator=g4, device=dev) * 0.02).to(torch.bfloat16)
        cap4 = gg.route_rows_bound(tokens4 * topk4, w4.num_groups, 16)
        ws4 = torch.empty(int(gg.load().gg_route_workspace_bytes(tokens4 * topk4, w4.num_groups)),
                          dtype=torch.uint8, device=dev)
        offs4 = torch.empty(w4.num_groups, dtype=torch.int32, device=dev)
        rs4 = torch.empty(cap4, dtype=torch.int32, device=dev)
        sr4 = torch.empty(tokens4 * topk4, dtype=torch.int32, device=dev)
        xg4 = torch.empty((cap4, w4.k), dtype=torch.bfloat16, device=dev)
        y4 = torch.empty((cap4, w4.n), dtype=torch.bfloat16, device=dev)
        o4 = torch.empty((tokens4, w4.n), dtype=torch.bfloat16, device=dev)
        bias4 = (torch.randn((w4.num_groups, w4.n), generator=g4, device=dev) * 0.1).to(torch.bfloat16)
        bscale4 = torch.rand((cap4,), generator=g4, device=dev)
        db4 = torch.empty((w4.num_groups, w4.n), dtype=torch.float32, device=dev)
        ds4 = torch.empty((cap4,), dtype=torch.float32, device=dev)
        st4 = torch.cuda.current_stream(dev).cuda_stream

        def route4():
            rc = gg.call_raw("gg_route", ids4.data_ptr(), tokens4 * topk4, w4.num_groups, 16, 1,
                             offs4.data_ptr(), rs4.data_ptr(), cap4, sr4.data_ptr(), ws4.data_ptr(), st4)
            assert rc == 0
        route4()
        _, ms4 = time_passes([("route", route4),
                              ("gather", lambda: gg.gather_rows(x4, rs4, topk4, offs4, out=xg4)),
                              ("forward", lambda: gg.forward(xg4, wt4, offs4, out=y4)),
                              ("forward_bias", lambda: gg.forward_bias(xg4, wt4, offs4, bias4, bscale4, out=y4)),
                              ("combine", lambda: gg.combine_rows(y4, sr4, topk4, probs4, out=o4)),
                              ("bias_grad", lambda: gg.bias_grad(y4, offs4, bscale4, out=db4)),
                              ("bias_scale_grad", lambda: gg.bias_scale_grad(y4, offs4, bias4, out=ds4))],
                             20, 3, torch)
        f4 = {k: sorted(v)[len(v) // 2] for k, v in ms4.items()}
        rows4 = int(offs4[-1].item())
        context["qwen3_routed_layer"] = {
            "tokens": tokens4, "topk": topk4, "experts": w4.num_groups, "min_alignment_m": 16,
            "padded_rows": rows4,
            "route_ms": round(f4["route"], 4),
            "gather_ms": round(f4["gather"], 4),
            "gather_GB/s": round(2 * rows4 * w4.k * 2 / (f4["gather"] * 1e-3) / 1e9, 1),
            "forward_ms": round(f4["forward"], 4),
            "forward_bias_scaled_ms": round(f4["forward_bias"], 4),
            "combine_ms": round(f4["combine"], 4),
            "combine_GB/s": round((tokens4 * topk4 * w4.n * 2 + tokens4 * w4.n * 2) / (f4["combine"] * 1e-3) / 1e9, 1),
            "bias_grad_ms": round(f4["bias_grad"], 4),
            "bias_grad_GB/s": round((rows4 * w4.n * 2 + rows4 * 4 + w4.num_groups * w4.n * 4)
                                    / (f4["bias_grad"] * 1e-3) / 1e9, 1),
            "bias_scale_grad_ms": round(f4["bias_scale_grad"], 4),
            "bias_scale_grad_GB/s": round((rows4 * w4.n * 2 + rows4 * 4 + w4.num_groups * w4.n * 2)
                                          / (f4["bias_scale_grad"] * 1e-3) / 1e9, 1)}
        del x4, wt4, xg4, y4, o4, ws4, rs4, sr4, db4, ds4
        torch.cuda.empty_cache()

        # fp8 (e4m3) block-scaled forward: the GLM-up and Qwen3 gate/up
        # recipes in fp8, and the masked down and gate/up projections of the
        # fp8 rollout (weights rotated over 3 copies as above).  The X-scale
        # packing, which a caller runs once per call, is timed on its own.
        for name in ("fp8_glm_up", "fp8_qwen3_gateup", "fp8_masked_down", "fp8_masked_gateup"):
            w8 = synth.by_name(name)
            t8 = synth.make_fp8_inputs(w8, dev)
            e8 = w8.num_groups
            masked = w8.layout == "masked"
            wsc = gg.fp8_pack_scales(gg.GG_FP8_WEIGHT, t8["sw"], None, w8.n, w8.k, e8)
            copies = 3 if masked else 1
            wq8 = [t8["w8"]] + [t8["w8"].clone() for _ in range(copies - 1)]
            grp = t8["masked_m"] if masked else t8["offs"]
            lay = gg.GG_FP8_ACT_MASKED if masked else gg.GG_FP8_ACT_RAGGED
            xsc = gg.fp8_pack_scales(lay, t8["sx"], grp, w8.m, w8.k, e8)
            y8 = torch.empty(((e8, w8.m, w8.n) if masked else (w8.m, w8.n)), dtype=torch.bfloat16, device=dev)
            r8 = {"i": 0}

            def wpick():
                r8["i"] = (r8["i"] + 1) % copies
                return wq8[r8["i"]]
            if masked:
                fwd8 = lambda: gg.fp8_masked_forward(t8["x8"], xsc, wpick(), wsc, grp, out=y8)
            else:
                fwd8 = lambda: gg.fp8_forward(t8["x8"], xsc, wpick(), wsc, grp, out=y8)
            pack8 = lambda: gg.fp8_pack_scales(lay, t8["sx"], grp, w8.m, w8.k, e8, out=xsc)
            reps = 10 if name == "fp8_glm_up" else 30
            _, ms8 = time_passes([("fwd", fwd8), ("pack", pack8)], reps, 3, torch)
            f8 = {k: sorted(v)[len(v) // 2] for k, v in ms8.items()}
            act = w8.active_rows()
            live8 = int((w8.group_sizes() > 0).sum())
            ab8 = act * w8.k + live8 * w8.n * w8.k + 2 * act * w8.n
            tf8 = w8.flops() / (f8["fwd"] * 1e-3) / 1e12
            gb8 = ab8 / (f8["fwd"] * 1e-3) / 1e9
            context[name] = {"fwd": {"ms": round(f8["fwd"], 4), "TFLOP/s": round(tf8, 2),
                                     "frac_of_fp8_mfma_peak": round(tf8 / PEAK_FP8_TFLOPS, 4),
                                     "algorithmic_GB/s": round(gb8, 1),
                                     "frac_of_hbm": round(gb8 / PEAK_HBM_GBS, 4)},
                             "pack_x_scales_ms": round(f8["pack"], 4)}
            if masked:
                context[name]["weights"] = "rotated over 3 copies (HBM-resident per call)"
            del t8, wq8, wsc, xsc, y8
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(wl, t, synth)

    out = {
        "metric": "grouped GEMM TFLOP/s (fwd/dgrad/wgrad) and % of bf16 MFMA peak, 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(secs / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "glm_up: 32 experts, 262144 rows (Dirichlet(1) sizes rounded to 128), "
                        "K=6144, N=4096; step = forward + dgrad + wgrad",
            "experts": wl.num_groups, "rows": wl.m, "k": wl.k, "n": wl.n,
            "outputs": "Y bf16, dX bf16, dW fp32",
            "flop_per_step": flop_step,
        },
        "frac_of_mfma_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "device": device_info(torch),
        "per_pass": per_pass,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "context": context,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
