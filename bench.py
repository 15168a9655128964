#!/usr/bin/env python3
"""WTConv training-step benchmark on one MI355X.

A step is one pass of the whole hot path over one batch, through the C-ABI,
on synthetic seeded inputs already resident in HBM: the forward (wtconv_fwd)
and the whole backward (wtconv_bwd: dx and every weight gradient in one call,
the library's fused backward). With --two-call-bwd the backward is
wtconv_bwd_data + wtconv_bwd_weight instead; the line reports that step's
time too, measured in the same run. The default workload is the largest single-GPU
configuration: B=16, C=256, 256x256, L=4, 7x7 base and 5x5 level kernels,
bf16 activations, fp32 arithmetic.

Prints one JSON line: images/s, the achieved HBM rate against the I/O-model
minimum bytes, the roofline of the dominant call (measured with HIP events
on the stream the kernels run on), the same figures for every other bar
workload (`workloads`), the naive unfused chain timed in the same run,
context lines (torch's own depthwise convolution of the same shape, and a
ConvNeXt-style block with WTConv, with torch's depthwise convolution and
with this library at L = 0 as its token mixer), the device's measured FMA
and copy rates, and the fp64 CPU oracle timed on a bounded sample on the
host.

Input sets are rotated so that their footprint exceeds 512 MiB: no step
finds its activations in the 256 MB last-level cache (MALL).

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "WTConv fwd+bwd images/sec and achieved HBM TB/s (% of MI355X peak)"
KERNEL_SOURCES = ("wtconv_device.h", "wtconv_plans.h", "wtconv_plane.h", "wtconv_fused.hip", "wtconv_tiled.h",
                  "wtconv_tiled.hip", "wtconv_bwdw.h", "wtconv_bwdw.hip", "wtconv_bwdw_body.h", "wtconv_dw.h",
                  "wtconv_dw.hip", "wtconv_api.hip", "wtconv_bwd1.h", "wtconv_bwd1.hip", "wtconv_family.h")
# rotated inputs must exceed twice the 256 MB MALL
ROTATION_BYTES = 512 << 20
# default warm-up before the timed steps
WARMUP_SECONDS = 0.3


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


def default_sets(cfg) -> int:
    """Input sets to rotate: at least two, and x + dy of all of them above
    ROTATION_BYTES."""
    per_set = 2 * cfg.N * (2 if cfg.dtype == "bf16" else 4)
    return max(2, math.ceil(ROTATION_BYTES / per_set) + 1)


def cpu_baseline(cfg, seconds: float):
    """The oracle as it stands, on the host cores, on the first images of the
    same workload; reported in images/s of the full three-call step."""
    import oracle
    from wavelet_convolution_amd.inputs import make_inputs

    nb = 2 if cfg.H * cfg.W * cfg.C <= (1 << 22) else 1
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
        "sample": f"{reps} x (fwd + bwd_data + bwd_weight) on the first {nb} image(s) "
                  f"({nb}x{cfg.C}x{cfg.H}x{cfg.W}) of {cfg.name}, fp64, {el:.1f} s",
    }


class Workload:
    """Device buffers of one workload: rotated input sets, parameters,
    outputs, gradients and one workspace for every call of a step."""

    def __init__(self, torch, wt, cfg, nsets: int, exact_first: bool, channels_last: bool = False):
        import numpy as np

        from wavelet_convolution_amd.inputs import make_inputs

        self.torch, self.wt, self.cfg = torch, wt, cfg
        dev = torch.device("cuda:0")
        act_dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        shape = (cfg.B, cfg.C, cfg.H, cfg.W)
        self.sets = []
        for s in range(nsets):
            if s == 0 and exact_first:
                # the seeded inputs the parity tests and the oracle use
                inp = make_inputs(cfg.B, cfg.C, cfg.H, cfg.W, cfg.L, cfg.kb, cfg.k, dtype=cfg.dtype, seed=0)

                def to_dev(a):
                    if cfg.dtype == "bf16":
                        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
                    return torch.from_numpy(a).to(dev)

                xs, dys = to_dev(inp.x), to_dev(inp.dy)
                self.wb = torch.from_numpy(inp.w_base).to(dev)
                self.wl = torch.from_numpy(inp.w_lvl).to(dev)
                self.sc = torch.from_numpy(inp.scale).to(dev)
                del inp
            else:
                # further sets of the same distributions, drawn on the device
                g = torch.Generator(device=dev)
                g.manual_seed(1000 + s)
                xs = torch.randn(shape, generator=g, device=dev).to(act_dt)
                dys = torch.randn(shape, generator=g, device=dev).to(act_dt)
                if s == 0:
                    self.wb = 0.02 * torch.randn(cfg.C, cfg.kb, cfg.kb, generator=g, device=dev)
                    self.wl = 0.02 * torch.randn(cfg.L, cfg.C, 4, cfg.k, cfg.k, generator=g, device=dev)
                    self.sc = 0.5 + torch.rand(cfg.L, cfg.C, 4, generator=g, device=dev)
            if channels_last:
                xs = xs.contiguous(memory_format=torch.channels_last)
                dys = dys.contiguous(memory_format=torch.channels_last)
            self.sets.append((xs, dys))
        self.y = torch.empty_like(self.sets[0][0])
        self.dx = torch.empty_like(self.sets[0][0])
        self.grads = (torch.empty((cfg.C, cfg.kb, cfg.kb), device=dev),
                      torch.empty(tuple(self.wl.shape), device=dev), torch.empty(tuple(self.sc.shape), device=dev))
        ws_bytes = max(wt.wtconv_workspace_size(self.sets[0][0], cfg.L, cfg.kb, cfg.k, op)
                       for op in (wt.OP_FWD, wt.OP_BWD_DATA, wt.OP_BWD_WEIGHT, wt.OP_BWD))
        self.ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)

    def step(self, i, single_pass=False, ev=None):
        wt, cfg = self.wt, self.cfg
        x, dy = self.sets[i % len(self.sets)]
        if ev is not None:
            ev[0].record()
        wt.wtconv_fwd(x, self.wb, self.wl, self.sc, y=self.y, ws=self.ws)
        if ev is not None:
            ev[1].record()
        if single_pass:
            # the whole backward in one call (events 1 -> 2 span it)
            wt.wtconv_bwd(x, dy, self.wb, self.wl, self.sc, dx=self.dx, out=self.grads, ws=self.ws)
            if ev is not None:
                ev[2].record()
        else:
            wt.wtconv_bwd_data(dy, self.wb, self.wl, self.sc, dx=self.dx, ws=self.ws)
            if ev is not None:
                ev[2].record()
            wt.wtconv_bwd_weight(x, dy, cfg.kb, self.wl, self.sc, out=self.grads, ws=self.ws)
        if ev is not None:
            ev[3].record()

    def time_steps(self, steps, run=None):
        """ms per step over `steps` steps bracketed by synchronisation."""
        torch = self.torch
        run = run or self.step
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            run(i)
        torch.cuda.synchronize()
        return 1e3 * (time.perf_counter() - t0) / steps

    def call_times(self, steps, single_pass=False):
        """Per-call durations (ms): HIP events on the stream the kernels run on."""
        torch = self.torch
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for i in range(steps):
            self.step(i, single_pass, evs[i])
        torch.cuda.synchronize()
        per = {"fwd": [], "bwd": []} if single_pass else {"fwd": [], "bwd_data": [], "bwd_weight": []}
        for e in evs:
            per["fwd"].append(e[0].elapsed_time(e[1]))
            if single_pass:
                per["bwd"].append(e[1].elapsed_time(e[2]))
            else:
                per["bwd_data"].append(e[1].elapsed_time(e[2]))
                per["bwd_weight"].append(e[2].elapsed_time(e[3]))
        mean = {k: sum(v) / len(v) for k, v in per.items()}
        med = {k: sorted(v)[len(v) // 2] for k, v in per.items()}
        return mean, med


def workload_summary(torch, wt, cfg, steps: int, single_pass: bool):
    """images/s, per-call times, step TFLOP/s and HBM rate of one bar
    workload (inputs drawn on the device, rotated above ROTATION_BYTES)."""
    from wavelet_convolution_amd import iomodel

    wl = Workload(torch, wt, cfg, default_sets(cfg), exact_first=False)
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < WARMUP_SECONDS or n < 10:   # the same warm-up as the main line
        for i in range(10):
            wl.step(n + i, single_pass)
        n += 10
        torch.cuda.synchronize()
    ms = wl.time_steps(steps, lambda i: wl.step(i, single_pass))
    mean, _ = wl.call_times(steps, single_pass)
    model = iomodel.step_model(cfg.B, cfg.C, cfg.H, cfg.W, cfg.L, cfg.kb, cfg.k, cfg.dtype)
    dominant = max(mean, key=mean.get)
    calls = 2 if dominant == "bwd" else 1
    step_bytes = model.step_bytes_fused_bwd if single_pass else model.step_bytes
    out = {"images_per_s": round(cfg.B / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
           "kernel_ms": {k: round(v, 5) for k, v in mean.items()},
           "step_TFLOPs": round(3 * model.flops_per_call / (ms * 1e-3) / 1e12, 2),
           "dominant": dominant,
           "dominant_frac_of_157TF": round(calls * model.flops_per_call / (mean[dominant] * 1e-3) / 1e12
                                           / iomodel.FP32_VECTOR_PEAK_TFLOPS, 4),
           "hbm_TBs_vs_min_bytes": round(step_bytes / (ms * 1e-3) / 1e12, 4),
           "input_sets_rotated": len(wl.sets), "steps": steps}
    del wl
    torch.cuda.empty_cache()
    return out


def depthwise_context(torch, wt, wl, steps: int):
    """The layer WTConv stands in for: a k_base x k_base depthwise convolution
    of the same activations, one step = forward + input gradient + weight
    gradient, timed two ways: through torch (MIOpen), with weights in the
    activations' dtype as torch requires (a library's kernels, not this
    package's), and through this library at L = 0 (its own depthwise kernels,
    the same three entry points with no levels)."""
    F = torch.nn.functional
    cfg, sets = wl.cfg, wl.sets
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
    y, dx = wl.y, wl.dx
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
        return wl.time_steps(steps, step)

    ms, own, own1 = timed(torch_step), timed(own_step), timed(own_single_pass)
    return {"what": f"depthwise conv {cfg.kb}x{cfg.kb}, fwd + input grad + weight grad", "ms_per_step": round(ms, 4),
            "images_per_s": round(cfg.B / (ms * 1e-3), 1), "steps": steps,
            "this_library_L0_ms_per_step": round(own, 4),
            "this_library_L0_single_pass_bwd_ms_per_step": round(own1, 4)}


def block_context(torch, wt, cfg, steps: int):
    """A ConvNeXt-style block with three token mixers, forward + backward of
    the whole block (every parameter gets its gradient, and the input too):

        h = mixer(x); h = LayerNorm_C(h); h = Linear_{C->4C}(h); h = GELU(h);
        h = Linear_{4C->C}(h); out = x + h

    The mixers: this library's WTConv (L levels), torch's k_base x k_base
    depthwise convolution, and this library at L = 0 (the same depthwise
    convolution through its own kernels). bf16 activations and block weights;
    the WTConv parameters are fp32. The linear layers run on flattened 2-D
    rows (plain matrix products)."""
    import torch.nn.functional as F

    from wavelet_convolution_amd.module import wtconv

    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    B, C, H, W = cfg.B, cfg.C, cfg.H, cfg.W
    g = torch.Generator(device=dev)
    g.manual_seed(7)

    def param(*shape, std=0.02, dtype=dt):
        return (std * torch.randn(*shape, generator=g, device=dev)).to(dtype).requires_grad_(True)

    ln_w = torch.ones(C, device=dev, dtype=dt, requires_grad=True)
    ln_b = torch.zeros(C, device=dev, dtype=dt, requires_grad=True)
    w1, b1, w2, b2 = param(4 * C, C), param(4 * C), param(C, 4 * C), param(C)
    wt_wb = param(C, cfg.kb, cfg.kb, dtype=torch.float32)
    wt_wl = param(cfg.L, C, 4, cfg.k, cfg.k, dtype=torch.float32)
    wt_sc = (0.5 + torch.rand(cfg.L, C, 4, generator=g, device=dev)).requires_grad_(True)
    dw_w = param(C, 1, cfg.kb, cfg.kb)
    l0_wl = torch.empty(0, C, 4, cfg.k, cfg.k, device=dev)
    l0_sc = torch.empty(0, C, 4, device=dev)
    nsets = max(2, math.ceil(ROTATION_BYTES / (2 * cfg.N * (2 if dt == torch.bfloat16 else 4))))
    xs = [torch.randn(B, C, H, W, generator=g, device=dev).to(dt).requires_grad_(True) for _ in range(nsets)]
    gs = [torch.randn(B, C, H, W, generator=g, device=dev).to(dt) for _ in range(nsets)]

    mixers = {
        "wtconv": lambda x: wtconv(x, wt_wb, wt_wl, wt_sc),
        "torch_depthwise": lambda x: F.conv2d(x, dw_w, padding=cfg.kb // 2, groups=C),
        "this_library_L0": lambda x: wtconv(x, wt_wb, l0_wl, l0_sc),
    }

    def block(x, mixer):
        h = mixer(x)
        h = h.permute(0, 2, 3, 1).reshape(-1, C)
        h = F.layer_norm(h, (C,), ln_w, ln_b, eps=1e-6)
        h = F.gelu(F.linear(h, w1, b1))
        h = F.linear(h, w2, b2)
        return x + h.reshape(B, H, W, C).permute(0, 3, 1, 2)

    out = {"what": f"ConvNeXt-style block (mixer, LayerNorm, {C}->{4 * C}->{C} MLP with GELU, residual), "
                   f"{B}x{C}x{H}x{W} {cfg.dtype}, forward + backward", "steps": steps}
    for name, mixer in mixers.items():
        def step(i, mixer=mixer):
            x = xs[i % nsets]
            block(x, mixer).backward(gs[i % nsets])

        for i in range(2):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        out[f"{name}_ms_per_step"] = round(1e3 * (time.perf_counter() - t0) / steps, 4)
    out["wtconv_over_torch_depthwise"] = round(out["wtconv_ms_per_step"] / out["torch_depthwise_ms_per_step"], 3)
    out["wtconv_over_this_library_L0"] = round(out["wtconv_ms_per_step"] / out["this_library_L0_ms_per_step"], 3)
    del xs, gs
    torch.cuda.empty_cache()
    return out


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
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=None,
                    help=f"untimed warm-up steps (default: as many as fill {WARMUP_SECONDS} s)")
    ap.add_argument("--workload", default=None, help="workload name (default: the headline large-plane shape)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-naive", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay a HIP graph of each step instead of launching it from Python (measured "
                         "slower on this path: 0.19 vs 0.18 ms per stage-1 step)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the FMA-rate and copy-rate probes")
    ap.add_argument("--two-call-bwd", action="store_true",
                    help="run the backward as wtconv_bwd_data + wtconv_bwd_weight instead of one wtconv_bwd "
                         "call")
    ap.add_argument("--channels-last", action="store_true",
                    help="channels-last activations (planar kernels on converted copies)")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context lines: torch's depthwise convolution and the ConvNeXt-style block")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the brief timing of the other bar workloads")
    ap.add_argument("--no-other-form", action="store_true",
                    help="skip the timing of the other backward form (for profiled runs: only the measured "
                         "form's kernels then run)")
    ap.add_argument("--sets", type=int, default=None,
                    help="rotated input sets (default: enough that x and dy of all sets exceed 512 MiB)")
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
    from wavelet_convolution_amd import iomodel
    from wavelet_convolution_amd.configs import BAR_WORKLOADS, BLOCK_WORKLOAD, CONFIGS, HEADLINE

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    wt.load_library()
    cfg = CONFIGS[args.workload or HEADLINE]
    model = iomodel.step_model(cfg.B, cfg.C, cfg.H, cfg.W, cfg.L, cfg.kb, cfg.k, cfg.dtype)
    print(f"[bench] {cfg.describe()}", file=sys.stderr, flush=True)

    wl = Workload(torch, wt, cfg, args.sets or default_sets(cfg), exact_first=True,
                  channels_last=args.channels_last)

    single = not args.two_call_bwd

    def step(i):
        wl.step(i, single)

    # Warm-up: W untimed steps. By default W is what fills WARMUP_SECONDS
    # (the clocks take tens of milliseconds to settle; a block timed right
    # after a few steps runs about 5 % slow on the small workloads).
    if args.warmup is None:
        t0, args.warmup = time.perf_counter(), 0
        while time.perf_counter() - t0 < WARMUP_SECONDS or args.warmup < 10:
            for i in range(10):
                step(args.warmup + i)
            args.warmup += 10
            torch.cuda.synchronize()
    else:
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()

    # Optionally one HIP graph per input set holding the step's kernel
    # launches (the library allocates and memsets nothing, so the captured
    # step is the eager one).
    run = step
    if args.graph:
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        for s_ in range(len(wl.sets)):
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
    ms_per_step = wl.time_steps(args.steps, run)
    print(f"[bench] {ms_per_step:.4f} ms per step", file=sys.stderr, flush=True)

    # per-call durations: HIP events on the stream the kernels run on
    dur, med = wl.call_times(args.steps, single)
    dominant = max(dur, key=dur.get)
    calls = 2 if dominant == "bwd" else 1   # the whole backward does two calls' multiply-adds
    achieved = calls * model.flops_per_call / (dur[dominant] * 1e-3) / 1e12
    src_hash = kernel_source_hash()
    # the stored counter summaries are of planar runs
    traffic = None if args.channels_last else read_traffic(cfg.name, dominant, src_hash)

    # the other backward form, same inputs and run, as warm
    other = None
    if not args.no_other_form:
        for i in range(min(args.warmup, 100)):
            wl.step(i, not single)
        other_ms = wl.time_steps(args.steps, lambda i: wl.step(i, not single))
        other_mean, _ = wl.call_times(args.steps, not single)
        other = {"backward": "wtconv_bwd_data + wtconv_bwd_weight" if single else "wtconv_bwd",
                 "ms_per_step": round(other_ms, 4), "images_per_s": round(cfg.B / (other_ms * 1e-3), 1),
                 "kernel_ms": {k: round(v, 5) for k, v in other_mean.items()}}

    naive = None
    if not args.no_naive:
        nws = torch.empty(max(wt.wtconv_workspace_size(wl.sets[0][0], cfg.L, cfg.kb, cfg.k, op, naive=True)
                              for op in range(3)) + 256, dtype=torch.uint8, device=wl.y.device)

        def naive_step(i):
            x, dy = wl.sets[i % len(wl.sets)]
            wt.wtconv_naive_fwd(x, wl.wb, wl.wl, wl.sc, y=wl.y, ws=nws)
            wt.wtconv_naive_bwd_data(dy, wl.wb, wl.wl, wl.sc, dx=wl.dx, ws=nws)
            wt.wtconv_naive_bwd_weight(x, dy, cfg.kb, wl.wl, wl.sc, out=wl.grads, ws=nws)

        naive_step(0)
        nms = wl.time_steps(max(3, args.steps // 5), naive_step)
        naive = {"ms_per_step": round(nms, 4), "images_per_s": round(cfg.B / (nms * 1e-3), 1),
                 "fused_speedup": round(nms / ms_per_step, 3)}
        del nws
        torch.cuda.empty_cache()
        print("[bench] naive chain done", file=sys.stderr, flush=True)

    context = None
    if not args.no_context:
        context = depthwise_context(torch, wt, wl, max(5, args.steps // 4))
        context["wtconv_over_depthwise"] = round(ms_per_step / context["ms_per_step"], 3)
        context["wtconv_over_this_library_L0"] = round(ms_per_step / context["this_library_L0_ms_per_step"], 3)
        print("[bench] depthwise context done", file=sys.stderr, flush=True)

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=wl.y.device).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1.0, out=dst)   # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    config = {"workload": cfg.name, "B": cfg.B, "C": cfg.C, "H": cfg.H, "W": cfg.W, "levels": cfg.L,
              "k_base": cfg.kb, "k_level": cfg.k, "activations": cfg.dtype, "parameters": "f32",
              "accumulate": "f32", "input_sets_rotated": len(wl.sets),
              "rotated_footprint_MB": round(len(wl.sets) * 2 * cfg.N * (2 if cfg.dtype == "bf16" else 4) / 1e6, 1),
              "launch": "hip graph per step" if args.graph else "eager",
              "layout": "channels_last" if args.channels_last else "nchw",
              "backward": "wtconv_bwd" if single else "wtconv_bwd_data + wtconv_bwd_weight"}
    del wl
    torch.cuda.empty_cache()

    block = None
    if not args.no_context:
        block = block_context(torch, wt, CONFIGS[BLOCK_WORKLOAD], max(5, args.steps // 2))
        print("[bench] block context done", file=sys.stderr, flush=True)

    workloads = None
    if not args.no_workloads:
        workloads = {}
        for name in BAR_WORKLOADS:
            if name == cfg.name:
                continue
            workloads[name] = workload_summary(torch, wt, CONFIGS[name], max(10, args.steps), single)
            print(f"[bench] workload {name}: {workloads[name]['images_per_s']} images/s", file=sys.stderr,
                  flush=True)

    peaks = None if args.no_peaks else measure_peaks(torch, wt)

    step_s = ms_per_step * 1e-3
    min_bytes = model.step_bytes_fused_bwd if single else model.step_bytes
    hbm_tbs = min_bytes / step_s / 1e12
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
        # the arithmetic type: every product and sum is fp32 (activations are
        # stored as config.activations)
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
        "hbm": {"min_bytes_per_step": min_bytes, "achieved_TBs": round(hbm_tbs, 4),
                "frac_of_8TBs": round(hbm_tbs / iomodel.HBM_PEAK_TBS, 4)},
        "kernel_ms": {k: round(v, 5) for k, v in dur.items()},
        "kernel_ms_median": {k: round(v, 5) for k, v in med.items()},
        "roofline": {"bound": "alu", "kernel": dominant, "achieved": round(achieved, 3),
                     "peak": iomodel.FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / iomodel.FP32_VECTOR_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "flops_per_launch": calls * model.flops_per_call,
                     "unpacked_fma_ceiling_TFLOPs": iomodel.FP32_UNPACKED_FMA_TFLOPS},
        "other_backward_form": other,
        "workloads": workloads,
        "naive_baseline": naive,
        "context": context,
        "block_context": block,
        "peaks_measured": peaks,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
