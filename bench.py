#!/usr/bin/env python3
"""Benchmark of the fused ConvTranspose3d + epilogue path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole path over one batch of synthetic input that
is already resident in HBM: re-lay the weights for the matrix cores
(convt3d_prepack_weights), then convt3d_fused (convolution with the fused
epilogue, statistics, normalisation).  The headline workload is the largest
of the five configurations, x [8,128,32,32,32] -> ConvTranspose3d(128->128,
k4, s2, p1) -> ReLU -> GroupNorm(16) (the largest tensors; the k5 BatchNorm
layer has 2 % more multiply-adds and is reported beside it).  Every one of
the five configurations is measured the same way in the same run and
reported in ``all_configs``, each with the largest |error| of its output
against the fp64 oracle on the same inputs.

Before the warm-up the plan is chosen once by timing (convt3d_autotune, as a
caller would do once per geometry); ``--no-tune`` keeps the cost model's
plan, and ``--plan`` / ``--phase-loop`` force one (the ``plan_string`` the
output reports selects the timed plan again without tuning, e.g. for a
profiler run whose kernel list should hold only the timed launches).

Prints ONE JSON line.  ``value`` is algorithmic GFLOP/s = 2 * (multiply-adds
whose input voxel is in range) / time per step.  ``roofline`` describes the
dominant kernel (the convolution kernel, FP32 MFMA bound): its duration comes
from HIP events the library records on the launch stream over the timed
region.  ``cpu_baseline`` times the fp64 CPU oracle on the host cores; the
same oracle run gives ``max_abs_err`` of the timed plan's output.
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

PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense FP32 matrix peak
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
METRIC = "ConvTranspose3d+epilogue GFLOP/s and ms/forward; % FP32 MFMA peak"
CSRC = os.path.join(ROOT, "activation_epilogues_amd", "csrc")
# source file of each kernel a roofline line is given for
# the sources each profiled kernel's code is built from: its file and the
# headers whose code it inlines
KERNEL_SRC = {"convt3d_mfma_kernel": [os.path.join(CSRC, f) for f in
                                      ("kernels.hip", "conv_index.hpp", "convt3d_internal.hpp")],
              "eval_binsum_kernel": [os.path.join(CSRC, f) for f in
                                     ("epilogue.hip", "conv_index.hpp", "convt3d_internal.hpp")]}
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash(kernel: str = "convt3d_mfma_kernel") -> str:
    """Hash of the sources `kernel` is built from (in a fixed order)."""
    h = hashlib.sha256()
    for path in KERNEL_SRC[kernel]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kernel: str = "convt3d_mfma_kernel"):
    """(HBM bytes per launch, plan string) of `kernel` from the committed
    rocprofv3 --pmc summary, if it was taken from the current kernel source
    (else (None, None)).  The plan is the one the counters were read on (the
    --plan of the profiled command; None when it ran untuned)."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None, None
    kv, plan = {}, None
    for line in open(path):
        m = re.search(r"--plan (\S+)", line)
        if m and plan is None:
            plan = m.group(1)
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(kernel):
        return None, None
    try:
        return float(kv["hbm_bytes_per_launch"]), plan
    except (KeyError, ValueError):
        return None, None


def dense_equivalent(wl, out_dims, ms: float) -> dict:
    """The pages' way of counting the work, for context only: every output
    voxel times every input channel (of its group) times every kernel tap,
    as a direct convolution over a zero-inserted, zero-padded input would
    multiply (the p77 page's 424 G multiply-adds for its k5 layer)."""
    kd, kh, kw = wl.kdims
    S = out_dims[0] * out_dims[1] * out_dims[2]
    macs = wl.n * wl.cout * S * (wl.cin // wl.conv_groups) * kd * kh * kw
    return {"gmac_per_step": round(macs / 1e9, 3), "gflops": round(2 * macs / (ms * 1e-3) / 1e9, 1),
            "note": "context only: counts zero-inserted and padding taps, not work done"}


def torch_comparison(wl, call, x, w, b, gamma, beta, rmean, rvar, fused_ms, reps: int = 5):
    """Context only: PyTorch-ROCm's own ConvTranspose3d followed by its
    epilogue ops (eager), its conv alone, and its conv followed by
    convt3d_epilogue_only; each timed with events over `reps` calls after one
    warm-up call, plus the largest difference of the eager result from the
    fused one."""
    import torch
    import torch.nn.functional as F
    from activation_epilogues_amd import convt3d as C
    from activation_epilogues_amd import workloads as W
    torch.backends.cudnn.allow_tf32 = False   # keep fp32 arithmetic in the vendor conv
    torch.backends.cuda.matmul.allow_tf32 = False
    rm_t = None if rmean is None else rmean.clone()
    rv_t = None if rvar is None else rvar.clone()

    def conv():
        return F.conv_transpose3d(x, w, b, stride=W.triple(wl.stride), padding=W.triple(wl.pad),
                                  output_padding=W.triple(wl.out_pad), groups=wl.conv_groups,
                                  dilation=W.triple(wl.dilation))

    def tail(y):
        if wl.epi == W.EPI_RELU_GROUPNORM:
            return F.group_norm(F.relu(y), wl.groups, gamma, beta, eps=wl.eps)
        if wl.epi == W.EPI_SOFTMAX_SIGMOID:
            return torch.sigmoid(torch.softmax(y, dim=1))
        if wl.epi in (W.EPI_SCALE_BN_TRAIN_AVGPOOL, W.EPI_SCALE_BN_EVAL_AVGPOOL):
            training = wl.epi == W.EPI_SCALE_BN_TRAIN_AVGPOOL
            z = F.batch_norm(y * wl.scale, rm_t, rv_t, gamma, beta, training=training, momentum=wl.momentum,
                             eps=wl.eps)
            return F.adaptive_avg_pool3d(z, 1)
        return y

    S = int(call.out_dims[0] * call.out_dims[1] * call.out_dims[2])
    epi = C.make_epilogue(wl.epi, wl.groups, wl.eps, wl.scale, gamma, beta, None, wl.momentum, None, None)
    has_tail = wl.epi != W.EPI_NONE
    ws_bytes = C.convt3d_epilogue_workspace_size(wl.n, wl.cout, S, epi) if has_tail else 0
    ws = torch.empty(max(1, ws_bytes // 4), device=x.device)
    pooled = wl.epi in (W.EPI_SCALE_BN_TRAIN_AVGPOOL, W.EPI_SCALE_BN_EVAL_AVGPOOL)

    def conv_then_ours():
        y = conv()
        if not has_tail:
            return y
        out = torch.empty((wl.n, wl.cout), device=x.device) if pooled else y
        C.convt3d_epilogue_only(y, wl.n, wl.cout, S, epi, out, ws, ws_bytes)
        return out

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    print("[bench] timing the PyTorch comparison", file=sys.stderr, flush=True)
    eager_ms = timed(lambda: tail(conv()))
    conv_ms = timed(conv)
    ours_tail_ms = timed(conv_then_ours)
    ref = tail(conv()).reshape(call.out.shape)
    diff = float((ref - call.out).abs().max())
    res = {"torch_eager_ms": round(eager_ms, 3), "torch_conv_ms": round(conv_ms, 3),
           "torch_conv_plus_epilogue_only_ms": round(ours_tail_ms, 3), "fused_ms_per_step": round(fused_ms, 3),
           "speedup_vs_torch_eager": round(eager_ms / fused_ms, 2), "max_abs_diff_vs_torch_eager": diff,
           "reps": reps, "note": "PyTorch-ROCm (MIOpen) fp32, TF32 off; context only"}
    if has_tail:
        # convt3d_epilogue_only alone on a resident y: its passes move
        # (reads, writes) x |y| bytes: GN (2, 1), softmax (1, 1) up to 1024
        # channels (held in registers) else (2, 1), BN (1, 0)
        y = conv()
        out = torch.empty((wl.n, wl.cout), device=x.device) if pooled else torch.empty_like(y)
        ep_ms = timed(lambda: C.convt3d_epilogue_only(y, wl.n, wl.cout, S, epi, out, ws, ws_bytes))
        if pooled:
            passes = 1
        elif wl.epi == W.EPI_SOFTMAX_SIGMOID and wl.cout <= 1024:
            passes = 2
        else:
            passes = 3
        gbps = passes * 4.0 * y.numel() / (ep_ms * 1e-3) / 1e9
        res.update({"epilogue_only_ms": round(ep_ms, 4), "epilogue_only_GBps": round(gbps, 1),
                    "epilogue_only_frac_hbm": round(gbps / PEAK_HBM_GBS, 4),
                    "epilogue_only_y_passes": passes})
    return res


HEADLINE = "k4s2_gn"


def measure(wl, args, log=print):
    """Tune, warm up and time one workload; returns its result dict (the
    fields of the JSON line, without the top-level metric fields)."""
    import numpy as np
    import torch
    from activation_epilogues_amd import convt3d as C
    from activation_epilogues_amd import workloads as W

    inp = W.make_inputs(wl)
    dev = torch.device("cuda:0")
    g = C.make_geom(wl.n, wl.cin, wl.cout, wl.d, wl.h, wl.w, wl.k, wl.stride, wl.pad, wl.out_pad,
                    wl.dilation, wl.conv_groups)
    call = C.FusedCall(g, wl.epi, wl.groups, wl.eps, wl.scale, device=dev)
    x = torch.from_numpy(inp.x).to(dev)
    w = torch.from_numpy(inp.w).to(dev)
    b = None if inp.b is None else torch.from_numpy(inp.b).to(dev)
    gamma = None if inp.gamma is None else torch.from_numpy(inp.gamma).to(dev)
    beta = None if inp.beta is None else torch.from_numpy(inp.beta).to(dev)
    # BatchNorm running statistics (training: updated every step; eval: read)
    rmean = None if inp.rmean is None else torch.from_numpy(inp.rmean).to(dev)
    rvar = None if inp.rvar is None else torch.from_numpy(inp.rvar).to(dev)
    evalmode = wl.epi == W.EPI_SCALE_BN_EVAL_AVGPOOL
    stream = torch.cuda.current_stream()
    tune = None
    if not args.no_tune:
        call.prepack(w, stream)
        tune = call.autotune(x, b, gamma, beta, stream)
        log(f"[bench] {wl.name}: plan tuned: {tune}")
    info = call.plan_info()
    # the eval path runs no convolution; its throughput is quoted against the
    # multiply-adds of the convolution it replaces (same output)
    conv_macs = C.convt3d_get_plan_info(g, C.make_epilogue(W.EPI_NONE))["valid_macs"] if evalmode else \
        info["valid_macs"]
    flops = 2.0 * conv_macs

    def step():
        call.prepack(w, stream)
        call(x, b, gamma, beta, stream, running_mean=rmean, running_var=rvar)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {wl.name}: warmup done ({args.warmup} steps), timing {args.steps} steps")

    # per-step events on the launch stream give the median step time; the
    # library brackets only the dominant kernel (the roofline's) with HIP
    # events inside the timed region: an event pair around every kernel adds a
    # few microseconds to each step (1.4 % on k3s1_gn, 4 % on k3s2_softmax)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    C.convt3d_profile_begin_kinds(C.PROFILE_REDUCE if evalmode else C.PROFILE_CONV)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = C.convt3d_profile_end()
    ms = (t1 - t0) * 1e3 / args.steps
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    ms_median = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (
        step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])
    gflops = flops / (ms * 1e-3) / 1e9
    log(f"[bench] {wl.name}: timed region done: {ms:.3f} ms/step")
    # the output of the last timed step (every step computes the same output
    # from the same inputs; BatchNorm's running statistics do not enter it)
    out_gpu = call.out.detach().cpu().numpy().astype(np.float64)

    # per-kernel breakdown (context): the same steps again after the timed
    # region, every kernel bracketed
    C.convt3d_profile_begin()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof_all = C.convt3d_profile_end()

    calls = max(1, prof["calls"])
    conv_ms = prof["conv_ms"] / calls
    if evalmode:
        # dominant kernel: the bin sums of x, HBM bound (reads x once, writes
        # the per-chunk bin sums)
        red_ms = prof["reduce_ms"] / calls
        eg_bins = info["eval_bins"]
        alg_bytes = 4.0 * (x.numel() + call.ws_bytes / 4)
        gbps = alg_bytes / (red_ms * 1e-3) / 1e9
        traffic, _ = stored_traffic(wl.name, kernel="eval_binsum_kernel")
        roofline = {
            "kernel": "eval_binsum_kernel",
            "bound": "hbm",
            "achieved": round(gbps, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": alg_bytes,
            "avg_launch_ms": round(red_ms, 4),
            "bins_per_plane": eg_bins,
        }
    else:
        conv_tflops = flops / (conv_ms * 1e-3) / 1e12
        traffic, traffic_plan = stored_traffic(wl.name)
        roofline = {
            "kernel": "convt3d_mfma_kernel",
            "bound": "mfma",
            "achieved": round(conv_tflops, 3),
            "peak": PEAK_FP32_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(conv_tflops / PEAK_FP32_MFMA_TFLOPS, 4),
            "traffic": traffic,
            # plan the traffic counters were read on (this run's plan_string may
            # differ when autotuning picks another candidate within noise)
            "traffic_plan": traffic_plan,
            "algorithmic_flop_per_launch": flops,
            "avg_launch_ms": round(conv_ms, 4),
        }
    calls_all = max(1, prof_all["calls"])
    kernels = {k: round(prof_all[k] / calls_all, 4)
               for k in ("conv_ms", "finalize_ms", "normalize_ms", "reduce_ms", "prepack_ms")}
    kernels["pass"] = "second pass of the same steps, every kernel bracketed by HIP events"
    if prof_all["normalize_ms"] > 0:
        # the output pass moves |y| per read and per write: GroupNorm's
        # normalise and the softmax over up to 1024 channels (held in the
        # registers of one position group) read once and write once; the
        # softmax over more channels reads twice
        passes = 3 if (wl.epi == W.EPI_SOFTMAX_SIGMOID and wl.cout > 1024) else 2
        norm_bytes = passes * 4.0 * call.out.numel()
        kernels["normalize_GBps"] = round(norm_bytes / (kernels["normalize_ms"] * 1e-3) / 1e9, 1)
        kernels["normalize_frac_hbm"] = round(kernels["normalize_GBps"] / PEAK_HBM_GBS, 4)
        kernels["normalize_y_passes"] = passes

    comparison = torch_comparison(wl, call, x, w, b, gamma, beta, rmean, rvar, ms) if args.compare_torch else None

    graph_ms = None
    if args.graph:
        # the same step captured once on a side stream and replayed: no host
        # launch cost per kernel (the library enqueues kernels only)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        g_step = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g_step, stream=side):
                call.prepack(w, side)
                call(x, b, gamma, beta, side, running_mean=rmean, running_var=rvar)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            g_step.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g_step.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    del call, x, w, b, gamma, beta, rmean, rvar
    torch.cuda.empty_cache()

    # the fp64 oracle on the same inputs (the whole batch): CPU baseline time
    # and the largest |error| of the timed plan's output
    cpu = None
    max_abs_err = None
    if not args.no_cpu_baseline:
        log(f"[bench] {wl.name}: running the CPU oracle on the same inputs")
        import oracle
        oracle.build()
        t0 = time.perf_counter()
        ref = oracle.run_workload(wl, inp)
        dt = time.perf_counter() - t0
        max_abs_err = float(np.abs(out_gpu - ref.out.reshape(out_gpu.shape)).max())
        del ref
        cpu = {"value": round(flops / dt / 1e9, 3), "unit": "GFLOP/s", "cores": oracle.num_threads(),
               "kind": "oracle", "sample": f"all {wl.n} samples of {wl.name}, whole path (conv + epilogue), fp64",
               "seconds": round(dt, 3)}

    return {
        "value": round(gflops, 2),
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(ms_median, 4),
        "config": {"workload": wl.name, "x": list(wl.x_shape), "cout": wl.cout, "k": wl.k, "stride": wl.stride,
                   "pad": wl.pad, "out_pad": wl.out_pad, "bias": wl.bias, "dilation": wl.dilation,
                   "conv_groups": wl.conv_groups, "epilogue": W.EPI_NAMES[wl.epi], "groups": wl.groups,
                   "scale": wl.scale},
        "value_kind": ("conv-equivalent: 2 x the in-range multiply-adds of the ConvTranspose3d whose pooled, "
                       "eval-mode-normalised output this path computes without running it") if evalmode else
                      "algorithmic: 2 x in-range multiply-adds of the ConvTranspose3d run",
        "pct_fp32_mfma_peak_whole_step": None if evalmode else round(100 * gflops / 1e3 / PEAK_FP32_MFMA_TFLOPS, 2),
        "max_abs_err": max_abs_err,
        "tolerance": 1e-4,
        "dense_equivalent": dense_equivalent(wl, info_dims(wl), ms),
        "roofline": roofline,
        "kernels": kernels,
        "plan": {k: v for k, v in info.items()},
        "plan_string": C.plan_string(info),
        "tune": tune,
        "cpu_baseline": cpu,
        "torch_comparison": comparison,
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
    }


def measure_epilogue_only(wl, args, log=print):
    """The standalone epilogue (convt3d_epilogue_only) on a conv output of the
    workload's shape already in HBM (the fused path's own NONE output, so the
    values are the real y), written to a separate buffer; repeated calls.
    GroupNorm and softmax are also timed in place (out == y)."""
    import torch
    from activation_epilogues_amd import convt3d as C
    from activation_epilogues_amd import workloads as W
    inp = W.make_inputs(wl)
    dev = torch.device("cuda:0")
    g = C.make_geom(wl.n, wl.cin, wl.cout, wl.d, wl.h, wl.w, wl.k, wl.stride, wl.pad, wl.out_pad,
                    wl.dilation, wl.conv_groups)
    conv = C.FusedCall(g, W.EPI_NONE, device=dev)
    conv.prepack(torch.from_numpy(inp.w).to(dev))
    y = conv(torch.from_numpy(inp.x).to(dev), None if inp.b is None else torch.from_numpy(inp.b).to(dev))
    torch.cuda.synchronize()
    del conv
    S = int(y[0, 0].numel())
    pooled = wl.epi in (W.EPI_SCALE_BN_TRAIN_AVGPOOL, W.EPI_SCALE_BN_EVAL_AVGPOOL)
    out = torch.empty((wl.n, wl.cout), device=dev) if pooled else torch.empty_like(y)
    gamma = None if inp.gamma is None else torch.from_numpy(inp.gamma).to(dev)
    beta = None if inp.beta is None else torch.from_numpy(inp.beta).to(dev)
    rmean = None if inp.rmean is None else torch.from_numpy(inp.rmean).to(dev)
    rvar = None if inp.rvar is None else torch.from_numpy(inp.rvar).to(dev)
    epi = C.make_epilogue(wl.epi, wl.groups, wl.eps, wl.scale, gamma, beta, None, wl.momentum, rmean, rvar)
    ws_bytes = C.convt3d_epilogue_workspace_size(wl.n, wl.cout, S, epi)
    ws = torch.empty(max(1, ws_bytes // 4), device=dev)

    def call():
        C.convt3d_epilogue_only(y, wl.n, wl.cout, S, epi, out, ws, ws_bytes)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    C.convt3d_profile_begin()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    prof = C.convt3d_profile_end()
    # bytes the passes move, in units of |y|: GroupNorm reads y twice and
    # writes once; the softmax (up to 1024 channels) reads once and writes
    # once; the BatchNorm kinds read once
    if wl.epi == W.EPI_RELU_GROUPNORM:
        passes = 3
    elif wl.epi == W.EPI_SOFTMAX_SIGMOID:
        passes = 2 if wl.cout <= 1024 else 3
    else:
        passes = 1
    nbytes = passes * 4.0 * y.numel()
    gbps = nbytes / (ms * 1e-3) / 1e9
    kern = {k: round(prof[k] / args.steps, 4) for k in ("reduce_ms", "finalize_ms", "normalize_ms")}
    # each HBM pass on its own (its kernel's HIP-event time): the statistics
    # pass reads |y|; the output pass (GroupNorm's normalise, the softmax)
    # reads |y| (twice for the softmax above 1024 channels) and writes |y|
    pass_bytes = {"reduce_ms": 4.0 * y.numel(),
                  "normalize_ms": (passes - (1 if wl.epi == W.EPI_RELU_GROUPNORM else 0)) * 4.0 * y.numel()}
    per_pass = {}
    for k, b in pass_bytes.items():
        if kern[k] > 0:
            r = b / (kern[k] * 1e-3) / 1e9
            per_pass[k.replace("_ms", "")] = {"ms": kern[k], "GBps": round(r, 1), "frac_hbm": round(r / PEAK_HBM_GBS, 4)}
    log(f"[bench] {wl.name} epilogue only: {ms:.4f} ms/call, {gbps:.0f} GB/s; per pass {per_pass}")
    in_place = None
    if not pooled:
        # the same calls with out == y (the API allows it); y's values change
        # from call to call, its size and the work per call do not
        def call_in_place():
            C.convt3d_epilogue_only(y, wl.n, wl.cout, S, epi, y, ws, ws_bytes)

        for _ in range(args.warmup):
            call_in_place()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            call_in_place()
        e1.record()
        torch.cuda.synchronize()
        ms_ip = e0.elapsed_time(e1) / args.steps
        gbps_ip = nbytes / (ms_ip * 1e-3) / 1e9
        in_place = {"ms_per_call": round(ms_ip, 4), "value": round(gbps_ip, 1),
                    "frac_hbm": round(gbps_ip / PEAK_HBM_GBS, 4)}
        log(f"[bench] {wl.name} epilogue only, in place: {ms_ip:.4f} ms/call, {gbps_ip:.0f} GB/s")
    return {
        "metric": "convt3d_epilogue_only HBM rate on a resident conv output",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_call": round(ms, 4), "higher_is_better": True, "frac_hbm": round(gbps / PEAK_HBM_GBS, 4),
        "y_passes": passes, "bytes_per_call": nbytes, "kernels_ms": kern, "per_pass": per_pass,
        "in_place": in_place,
        "config": {"workload": wl.name, "y": list(y.shape), "epilogue": W.EPI_NAMES[wl.epi], "out": "separate buffer"},
        "dtype": "f32", "data": "the workload's own conv output (synthetic seeded inputs)",
    }


def info_dims(wl):
    """Output dims of a workload (for the dense-equivalent count)."""
    from activation_epilogues_amd import convt3d as C
    g = C.make_geom(wl.n, wl.cin, wl.cout, wl.d, wl.h, wl.w, wl.k, wl.stride, wl.pad, wl.out_pad,
                    wl.dilation, wl.conv_groups)
    return C.convt3d_output_dims(g)


def summary(r):
    """One config's line in all_configs."""
    k = r["kernels"]
    return {"ms_per_step": r["ms_per_step"], "gflops": r["value"],
            "conv_frac_fp32_mfma": None if r["roofline"]["bound"] != "mfma" else r["roofline"]["frac"],
            "conv_ms": r["roofline"]["avg_launch_ms"],
            "normalize_frac_hbm": k.get("normalize_frac_hbm"), "normalize_ms": k["normalize_ms"] or None,
            "max_abs_err": r["max_abs_err"],
            "oracle_s": None if r["cpu_baseline"] is None else r["cpu_baseline"]["seconds"],
            "plan_string": r["plan_string"], "workload": r["config"]["workload"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, help="the workload of the JSON line's headline fields")
    ap.add_argument("--only", action="store_true",
                    help="measure only --workload (default: also every one of the five configurations)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle (no CPU time, no max_abs_err)")
    ap.add_argument("--no-tune", action="store_true", help="keep the cost model's plan")
    ap.add_argument("--plan", default=None, help="force a plan (CONVT3D_PLAN string); implies --no-tune, --only")
    ap.add_argument("--phase-loop", type=int, choices=(0, 1), default=None,
                    help="force the phase-group loop off / on (with --plan)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a captured HIP graph (context; value stays eager)")
    ap.add_argument("--compare-torch", action="store_true",
                    help="also time PyTorch's own ConvTranspose3d + epilogue ops, and its conv followed by "
                         "convt3d_epilogue_only (context only)")
    ap.add_argument("--epilogue-only", action="store_true",
                    help="time convt3d_epilogue_only on the workload's conv output instead (its own JSON line)")
    args = ap.parse_args()
    if args.plan is not None:
        os.environ["CONVT3D_PLAN"] = args.plan
        args.no_tune = True
        args.only = True
    if args.phase_loop is not None:
        os.environ["CONVT3D_PHASE_LOOP"] = str(args.phase_loop)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(a batch split with one all-reduce of the BatchNorm sums is the design); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch  # noqa: F401  (loads torch's HIP runtime before the library)
    from activation_epilogues_amd import workloads as W

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    if args.epilogue_only:
        print(json.dumps(measure_epilogue_only(W.BY_NAME[args.workload], args, log)), flush=True)
        return
    head = measure(W.BY_NAME[args.workload], args, log)
    all_configs = None
    if not args.only:
        all_configs = {}
        for wl in W.WORKLOADS:
            r = head if wl.name == args.workload else measure(wl, args, log)
            all_configs[wl.name] = summary(r)
    res = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "ms_per_step_median": head["ms_per_step_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) input, U(+-1/sqrt(cin*k^3)) weights)",
    }
    res.update({k: v for k, v in head.items() if k not in res})
    res["all_configs"] = all_configs
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
