#!/usr/bin/env python3
"""WTConv training-step benchmark on one MI355X.

A step is one pass of the whole hot path over one batch: forward
(wtconv_fwd), backward data (wtconv_bwd_data) and backward weight
(wtconv_bwd_weight), each through the C-ABI, on synthetic seeded inputs
already resident in HBM. The default workload is the ConvNeXt stage-1 shape
(B=64, C=96, 56x56, L=3, 5x5 kernels, bf16 activations, fp32 arithmetic).

Prints one JSON line: images/s, the achieved HBM rate against the I/O-model
minimum bytes, the roofline of the dominant kernel (measured with HIP events
on the stream the kernels run on), the naive unfused chain timed in the same
run, torch's own depthwise convolution of the same shape as context, the
device's measured FMA and copy rates, and the fp64 CPU oracle timed on a
bounded sample on the host.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "WTConv fwd+bwd images/sec and achieved HBM TB/s (% of MI355X peak)"
KERNEL_SOURCES = ("wtconv_device.h", "wtconv_plans.h", "wtconv_plane.h", "wtconv_fused.hip", "wtconv_tiled.hip",
                  "wtconv_bwdw.hip", "wtconv_dw.h", "wtconv_dw.hip")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "wavelet_convolution_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, kernel: str, src_hash: str):
    """Per-launch HBM bytes of `kernel` from the committed counter summary,
    or None when there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_src_sha") != src_hash:
        return None
    try:
        return float(vals[f"{kernel}_hbm_bytes_per_launch"])
    except KeyError:
        return None


def cpu_baseline(cfg, seconds: float):
    """The oracle as it stands, on the host cores, on the first images of the
    same workload; reported in images/s of the full three-call step."""
    import numpy as np

    import oracle
    from wavelet_convolution_amd.inputs import make_inputs

    nb = 2
    inp = make_inputs(nb, cfg.C, cfg.H, cfg.W, cfg.L, cfg.kb, cfg.k, dtype=cfg.dtype, seed=0)
    x, dy = inp.act_f64("x"), inp.act_f64("dy")
    wb, wl, sc = inp.params_f64()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.fwd(x, wb, wl, sc)
        oracle.bwd_data(dy, wb, wl, sc)
        oracle.bwd_weight(x, dy, wb, wl, sc)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {
        "value": reps * nb / el,
        "unit": "images/s",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": f"{reps} x (fwd + bwd_data + bwd_weight) on the first {nb} images "
                  f"({nb}x{cfg.C}x{cfg.H}x{cfg.W}) of {cfg.name}, fp64, {el:.1f} s",
    }


def depthwise_context(torch, wt, cfg, sets, steps: int):
    """The layer WTConv stands in for: a k_base x k_base depthwise convolution
    of the same activations, one step = forward + input gradient + weight
    gradient, timed two ways: through torch (MIOpen), with weights in the
    activations' dtype as torch requires (a library's kernels, not this
    package's), and through this library at L = 0 (its own depthwise kernels,
    the same three entry points with no levels)."""
    F = torch.nn.functional
    dev = sets[0][0].device
    wdt = sets[0][0].dtype
    w = torch.randn(cfg.C, 1, cfg.kb, cfg.kb, device=dev).to(wdt)
    pad = cfg.kb // 2

    def torch_step(i):
        x, dy = sets[i % len(sets)]
        F.conv2d(x, w, padding=pad, groups=cfg.C)
        torch.ops.aten.convolution_backward(dy, x, w, None, [1, 1], [pad, pad], [1, 1], False, [0, 0], cfg.C,
                                            [True, True, False])

    wb = w.float().reshape(cfg.C, cfg.kb, cfg.kb).contiguous()
    wl0 = torch.empty(0, cfg.C, 4, cfg.k, cfg.k, device=dev)
    sc0 = torch.empty(0, cfg.C, 4, device=dev)
    y, dx = torch.empty_like(sets[0][0]), torch.empty_like(sets[0][0])
    grads = (torch.empty(cfg.C, cfg.kb, cfg.kb, device=dev), wl0, sc0)
    ws = torch.empty(max(wt.wtconv_workspace_size(sets[0][0], 0, cfg.kb, cfg.k, op) for op in range(4)) + 256,
                     dtype=torch.uint8, device=dev)

    def own_step(i):
        x, dy = sets[i % len(sets)]
        wt.wtconv_fwd(x, wb, wl0, sc0, y=y, ws=ws)
        wt.wtconv_bwd_data(dy, wb, wl0, sc0, dx=dx, ws=ws)
        wt.wtconv_bwd_weight(x, dy, cfg.kb, wl0, sc0, out=grads, ws=ws)

    def own_single_pass(i):
        x, dy = sets[i % len(sets)]
        wt.wtconv_fwd(x, wb, wl0, sc0, y=y, ws=ws)
        wt.wtconv_bwd(x, dy, wb, wl0, sc0, dx=dx, out=grads, ws=ws)

    def timed(step):
        for i in range(2):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        return 1e3 * (time.perf_counter() - t0) / steps

    ms, own, own1 = timed(torch_step), timed(own_step), timed(own_single_pass)
    return {"what": f"depthwise conv {cfg.kb}x{cfg.kb}, fwd + input grad + weight grad", "ms_per_step": round(ms, 4),
            "images_per_s": round(cfg.B / (ms * 1e-3), 1), "steps": steps,
            "this_library_L0_ms_per_step": round(own, 4),
            "this_library_L0_single_pass_bwd_ms_per_step": round(own1, 4)}


def measure_peaks(torch, wt, reps: int = 5):
    """The two ceilings on this device: unpacked fp32 FMA rate (probe kernel,
    16 independent chains per lane) and plain copy rate (1 GiB to 1 GiB).
    Best of `reps` timed launches each, HIP events on the current stream."""
    dev = torch.device("cuda:0")

    def best(fn):
        fn()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            work = fn()
            b.record()
            b.synchronize()
            ts.append((a.elapsed_time(b) * 1e-3, work))
        return min(ts)

    blocks, iters = 256 * 32, 2048
    out = torch.empty(blocks * 256, device=dev)
    t, flops = best(lambda: wt.wtconv_peak_fma(out, blocks, iters))
    src = torch.empty(1 << 28, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    tc, nbytes = best(lambda: wt.wtconv_peak_copy(src, dst))
    del out, src, dst
    return {"fma_f32_unpacked_TFLOPs": round(flops / t / 1e12, 2), "copy_TBs": round(nbytes / tc / 1e12, 3)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline stage-1 shape)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-naive", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay a HIP graph of each step instead of launching it from Python (measured "
                         "slower on this path: 0.19 vs 0.18 ms per stage-1 step)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the FMA-rate and copy-rate probes")
    ap.add_argument("--single-pass-bwd", action="store_true",
                    help="run the backward as one wtconv_bwd call (a single pass over x and dy where the "
                         "library has one: L = 0 on its planned planes)")
    ap.add_argument("--channels-last", action="store_true",
                    help="channels-last activations (planar kernels on converted copies)")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context line: torch's own depthwise convolution on the same shape")
    ap.add_argument("--sets", type=int, default=4, help="rotated input sets (defeats the 256 MB MALL)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the steps, copy one 1 GiB buffer (known HBM bytes) so that a counter "
                         "run can scale FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU layout is a design "
              "note (batch sharding plus one gradient all-reduce), not a measured path.", file=sys.stderr)
        return 2

    import torch

    from wavelet_convolution_amd import binding as wt
    from wavelet_convolution_amd.configs import CONFIGS, HEADLINE
    from wavelet_convolution_amd.inputs import make_inputs
    from wavelet_convolution_amd import iomodel

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    wt.load_library()
    cfg = CONFIGS[args.workload or HEADLINE]
    dev = torch.device("cuda:0")
    model = iomodel.step_model(cfg.B, cfg.C, cfg.H, cfg.W, cfg.L, cfg.kb, cfg.k, cfg.dtype)

    def to_dev(a):
        import numpy as np
        if cfg.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    sets = []
    for s in range(args.sets):
        inp = make_inputs(cfg.B, cfg.C, cfg.H, cfg.W, cfg.L, cfg.kb, cfg.k, dtype=cfg.dtype, seed=s)
        if s == 0:
            wb = torch.from_numpy(inp.w_base).to(dev)
            wl = torch.from_numpy(inp.w_lvl).to(dev)
            sc = torch.from_numpy(inp.scale).to(dev)
        xs, dys = to_dev(inp.x), to_dev(inp.dy)
        if args.channels_last:
            xs, dys = xs.contiguous(memory_format=torch.channels_last), dys.contiguous(memory_format=torch.channels_last)
        sets.append((xs, dys))
        del inp
    y = torch.empty_like(sets[0][0])
    dx = torch.empty_like(sets[0][0])
    grads = (torch.empty((cfg.C, cfg.kb, cfg.kb), device=dev), torch.empty(tuple(wl.shape), device=dev),
             torch.empty(tuple(sc.shape), device=dev))
    # one workspace for every call of a step, allocated before timing
    ws_bytes = max(wt.wtconv_workspace_size(sets[0][0], cfg.L, cfg.kb, cfg.k, op)
                   for op in (wt.OP_FWD, wt.OP_BWD_DATA, wt.OP_BWD_WEIGHT, wt.OP_BWD))
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)

    def step(i, ev=None):
        x, dy = sets[i % len(sets)]
        if ev is not None:
            ev[0].record()
        wt.wtconv_fwd(x, wb, wl, sc, y=y, ws=ws)
        if ev is not None:
            ev[1].record()
        if args.single_pass_bwd:
            # the whole backward in one call (events 1 -> 2 span it)
            wt.wtconv_bwd(x, dy, wb, wl, sc, dx=dx, out=grads, ws=ws)
            if ev is not None:
                ev[2].record()
        else:
            wt.wtconv_bwd_data(dy, wb, wl, sc, dx=dx, ws=ws)
            if ev is not None:
                ev[2].record()
            wt.wtconv_bwd_weight(x, dy, cfg.kb, wl, sc, out=grads, ws=ws)
        if ev is not None:
            ev[3].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Optionally one HIP graph per input set holding the step's four kernel
    # launches (the library allocates and memsets nothing, so the captured
    # step is the eager one).
    run = step
    if args.graph:
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        for s_ in range(len(sets)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(s_)
            graphs.append(g)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()

        def run(i):
            graphs[i % len(graphs)].replay()

        for i in range(len(graphs)):
            run(i)
        torch.cuda.synchronize()

    # whole-step timing: K steps bracketed by synchronisation
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps

    # per-kernel durations: HIP events on the stream the kernels run on
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    per = {"fwd": [], "bwd": []} if args.single_pass_bwd else {"fwd": [], "bwd_data": [], "bwd_weight": []}
    for e in evs:
        per["fwd"].append(e[0].elapsed_time(e[1]))
        if args.single_pass_bwd:
            per["bwd"].append(e[1].elapsed_time(e[2]))
        else:
            per["bwd_data"].append(e[1].elapsed_time(e[2]))
            per["bwd_weight"].append(e[2].elapsed_time(e[3]))
    dur = {k: sum(v) / len(v) for k, v in per.items()}   # mean ms per launch (the roofline's figure)
    med = {k: sorted(v)[len(v) // 2] for k, v in per.items()}
    dominant = max(dur, key=dur.get)
    calls = 2 if dominant == "bwd" else 1   # the whole backward does two calls' multiply-adds
    achieved = calls * model.flops_per_call / (dur[dominant] * 1e-3) / 1e12
    src_hash = kernel_source_hash()
    # the stored counter summaries are of planar runs
    traffic = None if (args.channels_last or args.single_pass_bwd) else read_traffic(cfg.name, dominant, src_hash)

    naive = None
    if not args.no_naive:
        nws = torch.empty(max(wt.wtconv_workspace_size(sets[0][0], cfg.L, cfg.kb, cfg.k, op, naive=True)
                              for op in range(3)) + 256, dtype=torch.uint8, device=dev)

        def naive_step(i):
            x, dy = sets[i % len(sets)]
            wt.wtconv_naive_fwd(x, wb, wl, sc, y=y, ws=nws)
            wt.wtconv_naive_bwd_data(dy, wb, wl, sc, dx=dx, ws=nws)
            wt.wtconv_naive_bwd_weight(x, dy, cfg.kb, wl, sc, out=grads, ws=nws)

        nsteps = max(3, args.steps // 5)
        naive_step(0)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(nsteps):
            naive_step(i)
        torch.cuda.synchronize()
        nms = 1e3 * (time.perf_counter() - t1) / nsteps
        naive = {"ms_per_step": round(nms, 4), "images_per_s": round(cfg.B / (nms * 1e-3), 1),
                 "fused_speedup": round(nms / ms_per_step, 3)}
        del nws

    context = None
    if not args.no_context:
        context = depthwise_context(torch, wt, cfg, sets, max(5, args.steps // 5))
        context["wtconv_over_depthwise"] = round(ms_per_step / context["ms_per_step"], 3)
        context["wtconv_over_this_library_L0"] = round(ms_per_step / context["this_library_L0_ms_per_step"], 3)

    peaks = None if args.no_peaks else measure_peaks(torch, wt)

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1.0, out=dst)   # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    step_s = ms_per_step * 1e-3
    hbm_tbs = model.step_bytes / step_s / 1e12
    out = {
        "metric": METRIC,
        "value": round(cfg.B / step_s, 1),
        "unit": "images/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "C": cfg.C, "H": cfg.H, "W": cfg.W, "levels": cfg.L,
                   "k_base": cfg.kb, "k_level": cfg.k, "activations": cfg.dtype, "accumulate": "f32",
                   "input_sets_rotated": len(sets), "launch": "hip graph per step" if args.graph else "eager",
                   "layout": "channels_last" if args.channels_last else "nchw",
                   "backward": "wtconv_bwd" if args.single_pass_bwd else "wtconv_bwd_data + wtconv_bwd_weight"},
        "hbm": {"min_bytes_per_step": model.step_bytes, "achieved_TBs": round(hbm_tbs, 4),
                "frac_of_8TBs": round(hbm_tbs / iomodel.HBM_PEAK_TBS, 4)},
        "kernel_ms": {k: round(v, 5) for k, v in dur.items()},
        "kernel_ms_median": {k: round(v, 5) for k, v in med.items()},
        "roofline": {"bound": "alu", "kernel": dominant, "achieved": round(achieved, 3),
                     "peak": iomodel.FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / iomodel.FP32_VECTOR_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "flops_per_launch": calls * model.flops_per_call,
                     "unpacked_fma_ceiling_TFLOPs": iomodel.FP32_UNPACKED_FMA_TFLOPS},
        "naive_baseline": naive,
        "context": context,
        "peaks_measured": peaks,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
