#!/usr/bin/env python3
"""Benchmark of the fused 3x3 conv + epilogue kernels on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the fused op over the whole batch of the workload
(inputs already resident in device memory).  The default workload is the
largest one: the 64->128 conv on x [64,64,256,256] with the x2.0 -> channel-min
epilogue (608.8 GFLOP per step).  Prints ONE JSON line on stdout.

Timing: W untimed warm-up steps, then exactly K steps bracketed by
torch.cuda.synchronize() on both sides (wall clock -> ms_per_step).  HIP
events recorded on the launch stream around the same K launches give the
per-launch kernel duration used for the roofline figure (also given as a
fraction of the MFMA-loop probe's throughput measured in the same run).  The other four
workloads are timed before the headline one (unless --no-others), which
also brings the GPU clocks to steady state first.  Every timing other than
the headline's warms up for at least WARM_S seconds of its own work: after
an idle spell, or on freshly allocated buffers, the first ~20 ms of work run
up to 15 % slower, which a fixed count of short launches does not cover.
All oracle comparisons run after the GPU timing, so that no timed workload
follows an idle GPU.

The CPU baseline is the oracle (test infrastructure) timed on a bounded
batch slice of the same workload on the host cores (by default the whole
batch of the headline workload); the GPU result for that slice is compared
with it element by element (max-abs error under "parity").  Every other
timed workload, and every NHWC form, is compared with the oracle on sampled
outputs (under "parity" of its own entry).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused conv3x3+epilogue ms/iter & effective TFLOP/s (% fp32 MFMA peak)"
PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix peak (AMD spec)
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E (AMD spec)
WARM_S = 0.25                   # minimum warm-up wall time of the non-headline timings


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "x3_conv2d_epilogue_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload: str):
    """HBM bytes per launch measured with rocprofv3 --pmc (FETCH_SIZE,
    WRITE_SIZE), stored in profiles/traffic.json together with the hash of
    the kernel sources they were taken on; None if absent or stale."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    e = d.get("workloads", {}).get(workload)
    if not e or d.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return e


def make_op(x3, wl, g, out=None, workspace=None):
    p = wl.params
    if wl.op == "min_tanh2":
        return lambda: x3.conv3x3_min_tanh2(g["x"], g["weight"], g["bias"], out=out)
    if wl.op == "scale_min":
        return lambda: x3.conv3x3_scale_min(g["x"], g["weight"], g["bias"], p["scale"], out=out)
    if wl.op == "mul_lrelu_gelu":
        return lambda: x3.conv3x3_mul_lrelu_gelu(g["x"], g["weight"], g["bias"], g["multiplier"],
                                                 p["neg_slope"], out=out)
    if wl.op == "gn_scale_pool_clamp":
        return lambda: x3.conv3x3_gn_scale_pool_clamp(
            g["x"], g["weight"], g["bias"], g["gamma"], g["beta"], g["scale"], p["groups"],
            p["eps"], p["pool_k"], p["lo"], p["hi"], out=out, workspace=workspace)
    raise ValueError(wl.op)


def split_ops(x3, wl, g, y, out):
    """The unfused form of a workload: (conv op writing y, epilogue op on y)."""
    p = wl.params
    conv = lambda: x3.conv3x3_bias(g["x"], g["weight"], g["bias"], out=y)  # noqa: E731
    if wl.op == "min_tanh2":
        epi = lambda: x3.epi_min_tanh2(y, out=out)  # noqa: E731
    elif wl.op == "scale_min":
        epi = lambda: x3.epi_scale_min(y, p["scale"], out=out)  # noqa: E731
    elif wl.op == "mul_lrelu_gelu":
        epi = lambda: x3.epi_mul_lrelu_gelu(y, g["multiplier"], p["neg_slope"], out=out)  # noqa: E731
    else:
        import torch  # noqa: PLC0415
        ws = torch.empty(x3.load_library().x3_epi_gn_workspace_bytes(wl.B, wl.Cout),
                         dtype=torch.uint8, device=y.device)
        epi = lambda: x3.epi_gn_scale_pool_clamp(  # noqa: E731
            y, g["gamma"], g["beta"], g["scale"], p["groups"], p["eps"], p["pool_k"], p["lo"],
            p["hi"], out=out, workspace=ws)
    return conv, epi


def epilogue_bytes(wl) -> int:
    """Algorithmic HBM bytes of a standalone epilogue: y read once, the
    output written once, per-channel vectors read once."""
    y = wl.B * wl.Cout * wl.Ho * wl.Wo
    n_out = 1
    for d in out_shape(wl):
        n_out *= d
    n_par = {"mul_lrelu_gelu": wl.Cout, "gn_scale_pool_clamp": 3 * wl.Cout}.get(wl.op, 0)
    return 4 * (y + n_out + n_par)


def ablation(torch, x3, wl, dev, steps, warmup, fused_ms):
    """Time the split path (conv storing y, then the standalone epilogue)
    against the fused kernel on the same workload."""
    g = gpu_inputs(torch, wl, dev, seed=0)
    y = torch.empty((wl.B, wl.Cout, wl.Ho, wl.Wo), device=dev)
    out = torch.empty(out_shape(wl), device=dev)
    conv, epi = split_ops(x3, wl, g, y, out)
    _, conv_ms = time_op(torch, conv, steps, warmup, WARM_S)
    _, epi_ms = time_op(torch, epi, steps, warmup, WARM_S)
    _, split_ms = time_op(torch, lambda: (conv(), epi()), steps, warmup, WARM_S)
    eb = epilogue_bytes(wl)
    gbps = eb / (epi_ms * 1e-3) / 1e9
    del g, y, out
    torch.cuda.empty_cache()
    return {"fused_kernel_ms": round(fused_ms, 4), "conv_store_ms": round(conv_ms, 4),
            "epilogue_ms": round(epi_ms, 4), "split_ms": round(split_ms, 4),
            "fused_speedup": round(split_ms / fused_ms, 3),
            "epilogue_bytes": eb, "epilogue_GBps": round(gbps, 1),
            "epilogue_frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4)}


def out_shape(wl):
    if wl.op in ("min_tanh2", "scale_min"):
        return (wl.B, 1, wl.Ho, wl.Wo)
    if wl.op == "mul_lrelu_gelu":
        return (wl.B, wl.Cout, wl.Ho, wl.Wo)
    k = wl.params["pool_k"]
    return (wl.B, wl.Cout, (wl.Ho - k) // k + 1, (wl.Wo - k) // k + 1)


def algorithmic_bytes(wl) -> int:
    """x read once + weights + bias + per-channel params + output written."""
    n_out = math.prod(out_shape(wl))
    n_par = {"mul_lrelu_gelu": 1, "gn_scale_pool_clamp": 3}.get(wl.op, 0) * wl.Cout
    return 4 * (wl.B * wl.Cin * wl.H * wl.W + wl.Cout * wl.Cin * 9 + wl.Cout + n_par + n_out)


def time_op(torch, op, steps, warmup, min_warm_s=0.0):
    """Wall-clock and HIP-event ms per launch of op over `steps` launches,
    after `warmup` untimed launches (and, given min_warm_s, untimed launches
    until that much wall time of them has completed)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        op()
    torch.cuda.synchronize()
    if min_warm_s > 0:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < min_warm_s:
            for _ in range(8):
                op()
            torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        op()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, ev0.elapsed_time(ev1) / steps


def graph_ms_per_call(torch, op, calls=20, replays=20):
    """Per-call time of `op` replayed from a HIP graph of `calls` back-to-back
    calls (no host launch work per call): for launch-bound workloads."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        op()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            op()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(replays):
        g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / (replays * calls)


def mfma_loop(torch, x3, dev):
    """The practical fp32 matrix-core ceiling on this GPU: the library's
    MFMA-loop probe (one 4-wave workgroup per CU, 8 independent
    32x32x2 fp32 MFMA chains per wavefront, no memory traffic), timed like
    the workloads; its outputs have a closed form (256 * iters)."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    n_out, iters = cus * 256, 8192
    out = torch.empty(n_out, device=dev)
    _, ms = time_op(torch, lambda: x3.probe_mfma(out, iters), 10, 3, WARM_S)
    tf = x3.probe_mfma_flop(n_out, iters) / (ms * 1e-3) / 1e12
    return {"tflops": round(tf, 2), "frac_peak": round(tf / PEAK_FP32_MFMA_TFLOPS, 4),
            "exact": bool((out == 256.0 * iters).all().item()), "kernel_ms": round(ms, 4),
            "workgroups": cus, "iters": iters}


def gpu_inputs(torch, wl, dev, seed=0, cpu_inputs=None):
    """Device-resident inputs.  Given CPU inputs (the seeded generator), copy
    them; otherwise draw the same distributions directly on the device."""
    if cpu_inputs is not None:
        return {k: v.to(dev) for k, v in cpu_inputs.items()}
    g = torch.Generator(device=dev).manual_seed(seed)
    a = 1.0 / math.sqrt(wl.Cin * 9)
    d = {"x": torch.randn((wl.B, wl.Cin, wl.H, wl.W), generator=g, device=dev),
         "weight": torch.empty((wl.Cout, wl.Cin, 3, 3), device=dev).uniform_(-a, a, generator=g),
         "bias": torch.empty((wl.Cout,), device=dev).uniform_(-a, a, generator=g)}
    if wl.op == "mul_lrelu_gelu":
        d["multiplier"] = 1 + 0.1 * torch.randn((wl.Cout,), generator=g, device=dev)
    if wl.op == "gn_scale_pool_clamp":
        d["gamma"] = 1 + 0.1 * torch.randn((wl.Cout,), generator=g, device=dev)
        d["beta"] = 0.1 * torch.randn((wl.Cout,), generator=g, device=dev)
        d["scale"] = 1 + 0.1 * torch.randn((wl.Cout,), generator=g, device=dev)
    return d


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo where there is one)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(wl, cpu_in, gpu_out, budget_s):
    """Time the oracle on a contiguous batch slice [0, b) of the workload,
    b chosen so the run takes about `budget_s` seconds; compare the GPU
    output on that slice."""
    import numpy as np
    import oracle

    def run(b):
        x = cpu_in["x"][:b].numpy()
        w, bias = cpu_in["weight"].numpy(), cpu_in["bias"].numpy()
        p = wl.params
        if wl.op == "min_tanh2":
            return oracle.min_tanh2(x, w, bias)
        if wl.op == "scale_min":
            return oracle.scale_min(x, w, bias, p["scale"])
        if wl.op == "mul_lrelu_gelu":
            return oracle.mul_lrelu_gelu(x, w, bias, cpu_in["multiplier"].numpy(), p["neg_slope"])
        return oracle.gn_scale_pool_clamp(x, w, bias, cpu_in["gamma"].numpy(),
                                          cpu_in["beta"].numpy(), cpu_in["scale"].numpy(),
                                          p["groups"], p["eps"], p["pool_k"], p["lo"], p["hi"])

    t0 = time.perf_counter()
    ref = run(1)
    t1 = time.perf_counter() - t0
    b = max(1, min(wl.B, int(budget_s / max(t1, 1e-3))))
    if b > 1:
        t0 = time.perf_counter()
        ref = run(b)
        dt = time.perf_counter() - t0
    else:
        dt = t1
    sub = wl.with_batch(b)
    got = gpu_out[:b].detach().cpu().numpy().astype(np.float64)
    err = float(np.abs(got - ref).max())
    return {
        "value": round(sub.conv_flops() / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"batch slice [0,{b}) of {wl.B} ({b * wl.Cin * wl.H * wl.W} input values), "
                  f"{dt:.2f} s wall; the full workload would take ~{dt * wl.B / b:.0f} s",
        "seconds": round(dt, 3),
    }, {"max_abs_err": err, "samples": b, "compared": int(got.size), "tolerance": 2e-4,
        "ok": err <= 2e-4, "kind": "whole batch" if b == wl.B else f"batch slice [0,{b})"}


def sampled_parity(wl, g, out, n=1500, seed=0):
    """Compare a timed output with the oracle on sampled elements: n random
    output pixels plus the first and last row and column of the first and
    last sample (all channels sampled at random for per-channel outputs);
    for the GroupNorm workload, two whole samples.  g and out are device
    tensors (either memory format); returns max-abs error and count."""
    import numpy as np
    import oracle

    c = {k: v.detach().cpu().contiguous().numpy() for k, v in g.items()}
    got = out.detach().cpu().contiguous().numpy().astype(np.float64)
    p = wl.params
    if wl.op == "gn_scale_pool_clamp":
        errs = []
        for b in sorted({0, wl.B - 1}):
            ref = oracle.gn_scale_pool_clamp(
                c["x"][b:b + 1], c["weight"], c["bias"], c["gamma"], c["beta"], c["scale"],
                p["groups"], p["eps"], p["pool_k"], p["lo"], p["hi"])
            errs.append(float(np.abs(got[b:b + 1] - ref).max()))
        err, cnt = max(errs), 2 * got[0].size
    else:
        rng = np.random.default_rng(seed)
        pts = [(b, r, q) for b in sorted({0, wl.B - 1}) for r in (0, wl.Ho - 1)
               for q in range(0, wl.Wo, max(1, wl.Wo // 16))]
        pts += [(b, r, q) for b in sorted({0, wl.B - 1}) for r in range(0, wl.Ho, max(1, wl.Ho // 16))
                for q in (0, wl.Wo - 1)]
        rnd = np.stack([rng.integers(0, wl.B, n), rng.integers(0, wl.Ho, n),
                        rng.integers(0, wl.Wo, n)], 1)
        pix = np.concatenate([np.array(pts, np.int64), rnd.astype(np.int64)])
        if wl.op == "mul_lrelu_gelu":
            co = rng.integers(0, wl.Cout, pix.shape[0])
            el = np.stack([pix[:, 0], co, pix[:, 1], pix[:, 2]], 1).astype(np.int64)
            ref = oracle.mul_lrelu_gelu_at(c["x"], c["weight"], c["bias"], c["multiplier"], el,
                                           p["neg_slope"])
            val = got[el[:, 0], el[:, 1], el[:, 2], el[:, 3]]
        elif wl.op == "scale_min":
            ref = oracle.scale_min_at(c["x"], c["weight"], c["bias"], pix, p["scale"])
            val = got[pix[:, 0], 0, pix[:, 1], pix[:, 2]]
        else:
            ref = oracle.min_tanh2_at(c["x"], c["weight"], c["bias"], pix)
            val = got[pix[:, 0], 0, pix[:, 1], pix[:, 2]]
        err, cnt = float(np.abs(val - ref).max()), int(pix.shape[0])
    return {"max_abs_err": err, "compared": cnt, "tolerance": 2e-4, "ok": err <= 2e-4,
            "kind": "sampled"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="scale_min")
    ap.add_argument("--cpu-budget", type=float, default=25.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--no-others", action="store_true",
                    help="do not time the other four workloads (the unfused and NHWC "
                         "comparisons then cover the chosen workload only)")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the unfused (conv + standalone epilogue) comparison")
    ap.add_argument("--no-nhwc", action="store_true",
                    help="skip timing the NHWC (channels_last) forms of the workloads")
    ap.add_argument("--copy-ref-mib", type=int, default=1024,
                    help="time a plain device-to-device copy of this size as the practical "
                         "HBM reference for the standalone epilogues (0 = skip)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on exactly one GPU (asked for {args.gpus}); "
              "the multi-GPU path is design-only (batch sharding, no collectives).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import x3_conv2d_epilogue_amd as x3
    from x3_conv2d_epilogue_amd.synthetic import WORKLOAD_ORDER, WORKLOADS, make_inputs

    x3.load_library()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    wl = WORKLOADS[args.workload]

    log(f"generating {wl.about} (seed 0, CPU)")
    cpu_in = make_inputs(wl, seed=0)
    # (sum, sum of magnitudes) of each input, in double: identifies the draw
    sums = {k: [round(float(v.sum(dtype=torch.float64)), 6),
                round(float(torch.linalg.vector_norm(v, 1, dtype=torch.float64)), 6)]
            for k, v in cpu_in.items()}
    g = gpu_inputs(torch, wl, dev, cpu_inputs=cpu_in)
    out = torch.empty(out_shape(wl), device=dev)
    ws = None
    if wl.op == "gn_scale_pool_clamp":
        p = wl.params
        ws = torch.empty(x3.gn_workspace_bytes(wl.B, wl.Cin, wl.H, wl.W, wl.Cout, p["groups"],
                                               p["pool_k"]), dtype=torch.uint8, device=dev)
    op = make_op(x3, wl, g, out=out, workspace=ws)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_probe_mib} MiB read + {args.copy_probe_mib} MiB written x3")

    # The other workloads are timed first: besides their own figures, they
    # bring the GPU to its steady-state clocks (after an idle spell the first
    # ~0.1 s of work runs several percent slower) before the headline run.
    # Their oracle comparisons wait in `pending` until all timing is done.
    others = {}
    pending = []
    if not args.no_others:
        for name in WORKLOAD_ORDER:
            if name == args.workload:
                continue
            w2 = WORKLOADS[name]
            g2 = gpu_inputs(torch, w2, dev, seed=0)
            o2 = torch.empty(out_shape(w2), device=dev)
            ws2 = None
            if w2.op == "gn_scale_pool_clamp":
                q = w2.params
                ws2 = torch.empty(x3.gn_workspace_bytes(w2.B, w2.Cin, w2.H, w2.W, w2.Cout,
                                                        q["groups"], q["pool_k"]),
                                  dtype=torch.uint8, device=dev)
            op2 = make_op(x3, w2, g2, out=o2, workspace=ws2)
            steps2 = max(3, min(args.steps, 20))
            mw, mk = time_op(torch, op2, steps2, max(1, args.warmup), WARM_S)
            f2 = w2.conv_flops()
            others[name] = {
                "about": w2.about, "ms_per_step": round(mw, 4), "kernel_ms": round(mk, 4),
                "tflops": round(f2 / (mk * 1e-3) / 1e12, 3),
                "frac_fp32_mfma_peak": round(f2 / (mk * 1e-3) / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4),
                "steps": steps2,
            }
            if w2.B * w2.Cout < 1024:
                # launch-bound: the same call replayed from a HIP graph
                gm = graph_ms_per_call(torch, op2)
                others[name]["graph_ms_per_call"] = round(gm, 4)
                others[name]["graph_tflops"] = round(f2 / (gm * 1e-3) / 1e12, 3)
            if args.cpu_budget > 0:
                pending.append((others[name], w2, g2, o2, 1500))
            del g2, o2, ws2, op2

    log(f"timing {args.workload}: warmup {args.warmup}, steps {args.steps}")
    ms_wall, ms_kernel = time_op(torch, op, args.steps, args.warmup)
    flops = wl.conv_flops()
    tflops = flops / (ms_wall * 1e-3) / 1e12
    achieved = flops / (ms_kernel * 1e-3) / 1e12

    # The practical MFMA ceiling, right after the headline timing.
    loop = mfma_loop(torch, x3, dev)

    traffic = load_traffic(args.workload)
    roof = {
        "bound": "mfma",
        "achieved": round(achieved, 3),
        "peak": PEAK_FP32_MFMA_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_FP32_MFMA_TFLOPS, 4),
        "traffic": traffic["bytes_per_launch"] if traffic else None,
        "kernel_ms": round(ms_kernel, 4),
        "frac_of_mfma_loop": round(achieved / loop["tflops"], 4),
        "algorithmic_flop_per_launch": flops,
        "algorithmic_bytes_per_launch": algorithmic_bytes(wl),
    }
    if wl.op == "gn_scale_pool_clamp":
        roof["note"] = "two kernels per launch (conv pass + finalize); kernel_ms covers both"

    # Unfused comparison: the same conv storing its output, then the
    # standalone epilogue kernel, per workload (after the headline timing).
    abl = {}
    if not args.no_ablation:
        fused = {args.workload: ms_kernel}
        fused.update({k: v["kernel_ms"] for k, v in others.items()})
        for name in WORKLOAD_ORDER:
            if name not in fused or WORKLOADS[name].B * WORKLOADS[name].Cout < 1024:
                continue  # (the tiny case says nothing about bandwidth)
            log(f"ablation {name}: conv + standalone epilogue")
            abl[name] = ablation(torch, x3, WORKLOADS[name], dev, max(3, min(args.steps, 20)),
                                 max(1, min(args.warmup, 5)), fused[name])

    # The NHWC (channels_last x) form of each workload, same values.
    nhwc = {}
    if not args.no_nhwc:
        for name in WORKLOAD_ORDER:
            w2 = WORKLOADS[name]
            if w2.B * w2.Cout < 1024 or (args.no_others and name != args.workload):
                continue
            log(f"nhwc {name}")
            g2 = gpu_inputs(torch, w2, dev, seed=0)
            g2["x"] = g2["x"].contiguous(memory_format=torch.channels_last)
            o2 = None
            if w2.op in ("mul_lrelu_gelu", "gn_scale_pool_clamp"):
                o2 = torch.empty(out_shape(w2), device=dev, memory_format=torch.channels_last)
            else:
                o2 = torch.empty(out_shape(w2), device=dev)
            ws2 = None
            if w2.op == "gn_scale_pool_clamp":
                q = w2.params
                ws2 = torch.empty(x3.gn_workspace_bytes(w2.B, w2.Cin, w2.H, w2.W, w2.Cout,
                                                        q["groups"], q["pool_k"], nhwc=True),
                                  dtype=torch.uint8, device=dev)
            op2 = make_op(x3, w2, g2, out=o2, workspace=ws2)
            steps2 = max(3, min(args.steps, 20))
            _, mk = time_op(torch, op2, steps2, max(1, min(args.warmup, 5)), WARM_S)
            f2 = w2.conv_flops()
            nhwc[name] = {"kernel_ms": round(mk, 4),
                          "tflops": round(f2 / (mk * 1e-3) / 1e12, 3),
                          "frac_fp32_mfma_peak": round(f2 / (mk * 1e-3) / 1e12 /
                                                       PEAK_FP32_MFMA_TFLOPS, 4)}
            if args.cpu_budget > 0:
                pending.append((nhwc[name], w2, g2, o2, 500))
            del g2, o2, ws2, op2

    # The practical HBM ceiling of a read+write stream on this machine: a plain
    # device-to-device copy (the runtime's copy kernel), large enough to
    # miss the 256 MB last-level cache.
    copy_ref = None
    if args.copy_ref_mib > 0:
        n = args.copy_ref_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        _, cms = time_op(torch, lambda: dst.copy_(src), 20, 3)
        gbps = 2 * 4 * n / (cms * 1e-3) / 1e9
        copy_ref = {"mib": args.copy_ref_mib, "ms": round(cms, 4), "GBps": round(gbps, 1),
                    "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4)}
        del src, dst
        torch.cuda.empty_cache()

    # Oracle comparisons of the other workloads and NHWC forms (host work).
    for entry, w2, g2, o2, n in pending:
        entry["parity"] = sampled_parity(w2, g2, o2, n=n)
    del pending
    torch.cuda.empty_cache()

    cpu = None
    parity = None
    if args.cpu_budget > 0:
        op()
        torch.cuda.synchronize()
        log(f"cpu baseline: oracle on the host cores (~{args.cpu_budget:.0f} s)")
        cpu, parity = cpu_baseline(wl, cpu_in, out, args.cpu_budget)

    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded: x~N(0,1), w,b~U(+-1/sqrt(Cin*9)))",
        "config": {"workload": wl.about, "x_shape": [wl.B, wl.Cin, wl.H, wl.W],
                   "cout": wl.Cout, "out_shape": list(out_shape(wl)), "seed": 0,
                   "flop_per_step": flops, "input_checksums": sums},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": parity,
        "other_workloads": others,
        "unfused_ablation": abl,
        "nhwc_workloads": nhwc,
        "copy_reference": copy_ref,
        "mfma_loop": loop,
        "host": {"cpu": cpu_model(), "cpu_count": os.cpu_count(),
                 "device": torch.cuda.get_device_name(0)},
    }
    if cpu:
        cpu["gpu_over_cpu"] = round(tflops / cpu["value"], 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
