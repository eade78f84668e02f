#!/usr/bin/env python3
"""Benchmark of the TTT forward scan on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

One step = one call of ttt_linear_fwd over the whole TTT-Linear 1.3B-layer
workload (B=4, H=32, T=8192, d=64, b=16, bf16 Q/K/V, fp32 eta / state / Z):
every stage of the scan (tile staging, projections, gradient, causal
attention-like mask, outputs, rank-b state update, final state) runs inside
the timed kernel.  Inputs are resident in HBM before timing starts.

Prints ONE JSON line: throughput in token*heads/s, the roofline of the scan
kernel (algorithmic bytes / measured kernel time vs 8 TB/s HBM), the fp64
oracle timed on the host cores as a baseline, and (unless --no-extras) the
other workloads: the b sweep, the 125M and long-context TTT-Linear shapes,
TTT-Linear with the LayerNorm + residual inner model (1.3B and 125M shapes),
TTT-MLP, the one-token decode steps of the three models, the forward with
checkpoints and the backward of TTT-Linear, the learning-rate gate and the
gated scan, and a streaming-copy bandwidth reference.

--pmc-calibrate additionally launches the streaming copy kernel on a known
byte count, so that a hardware-counter run of this script can scale the
scans' FETCH_SIZE / WRITE_SIZE readings (see --summarize-pmc), and the
LayerNorm and TTT-MLP scans, so that the same run covers every scan kernel.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, vendor figure
METRIC = "TTT fwd tokens·heads/s at 1 GPU; % of HBM/MFMA roofline (b=16)"
UNIT = "tokens·heads/s"
SCAN_SOURCES = ["ttt_linear_bf16.hip", "ttt_device.h", "ttt_launch.h", "ttt_linear_ops.h"]
LN_SOURCES = ["ttt_linear_ln.hip", "ttt_device.h", "ttt_launch.h", "ttt_linear_ops.h"]
MLP_SOURCES = ["ttt_mlp.hip", "ttt_mlp_ops.h", "ttt_device.h", "ttt_launch.h"]
MLP_BWD_SOURCES = ["ttt_mlp_bwd.hip", "ttt_mlp_ops.h", "ttt_device.h", "ttt_launch.h"]
LN_BWD_SOURCES = ["ttt_linear_ln_bwd.hip", "ttt_mlp_ops.h", "ttt_device.h", "ttt_launch.h"]
# kernel names as rocprofv3 reports them (the MLP scan's template arguments:
# waves, sub-batches, checkpoint stores, LayerNorm wrapper, held gradient point)
LN_SCAN_NAME = "linear_ln_scan_kernel<1, false, false>"  # one unit per workgroup, no checkpoint stores
MLP_SCAN_NAME = "mlp_scan_kernel<8, false, false, false, false>"
MLP_LN_SCAN_NAME = "mlp_scan_kernel<8, false, false, true, false>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
# untimed launches before each extra workload: the cache-flush writes of the
# headline's cold-start pass leave the clocks low for a few milliseconds
EXTRA_WARMUP = 50


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "test_rnn_layers_head_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# --------------------------------------------------------------------------
# algorithmic work per launch
# --------------------------------------------------------------------------
def linear_alg_bytes(wl) -> int:
    es = 2 if wl.qkv_dtype == "bf16" else 4
    per_tok = 3 * wl.d * es + 4 + wl.d * 4  # q, k, v in; eta in; z out (fp32)
    return wl.token_heads * per_tok + wl.H * wl.d * wl.d * 4 + wl.units * wl.d * wl.d * 4


def linear_alg_flops(wl, b) -> int:
    d = wl.d
    return wl.token_heads * (6 * d * d + 4 * b * d)


def ln_alg_bytes(wl) -> int:
    """The plain scan's bytes plus the LayerNorm scale and shift of each head."""
    return linear_alg_bytes(wl) + wl.H * wl.d * 2 * 4


def mlp_alg_bytes(wl) -> int:
    es = 2 if wl.qkv_dtype == "bf16" else 4
    per_tok = 3 * wl.d * es + 4 + wl.d * 4
    st = 2 * wl.hidden * wl.d * 4
    return wl.token_heads * per_tok + wl.H * st + wl.units * st


def mlp_ln_alg_bytes(wl) -> int:
    """The plain MLP scan's bytes plus the LayerNorm scale and shift of each head."""
    return mlp_alg_bytes(wl) + wl.H * wl.d * 2 * 4


def mlp_bwd_alg_bytes(wl, b=16) -> int:
    """TTT-MLP backward: q, k, v (bf16), eta, dz and the checkpoints in; dq,
    dk, dv, deta and both initial-state adjoints out."""
    nmb = (wl.T + b - 1) // b
    st = 2 * wl.hidden * wl.d * 4
    return wl.token_heads * (3 * wl.d * 2 + 4 + wl.d * 4 + 3 * wl.d * 4 + 4) + wl.units * (nmb + 1) * st


def ln_bwd_alg_bytes(wl, b=16) -> int:
    """TTT-Linear + LayerNorm backward: the plain backward's traffic (q, k,
    v, eta, dz and the checkpoints in; dq, dk, dv, deta and dW0 out) plus
    dgamma and dbeta per unit."""
    return bwd_alg_bytes(wl, b) + 2 * wl.units * wl.d * 4


def mlp_alg_flops(wl, b) -> int:
    d, h = wl.d, wl.hidden
    return wl.token_heads * (14 * h * d + 4 * b * (h + d))


# --------------------------------------------------------------------------
def device_inputs(x):
    import torch
    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    d = dict(q=dev(x.q_raw), k=dev(x.k_raw), v=dev(x.v_raw), eta=dev(x.eta))
    if x.w0 is not None:
        d["w0"] = dev(x.w0)
    else:
        d["w1"], d["w2"] = dev(x.w1), dev(x.w2)
    return d


_FLUSH = None


def flushed_launches(launch, reps):
    """Single-launch times (us) with a 512 MiB write before each launch, so
    that no input is left in the 256 MB MALL or the L2s: median, p10, p90."""
    import torch
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
    ks = []
    for i in range(reps):
        _FLUSH.fill_(float(i))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        launch()
        b.record()
        torch.cuda.synchronize()
        ks.append(a.elapsed_time(b) * 1e3)
    ks = np.array(ks)
    return {"median": float(np.median(ks)), "p10": float(np.percentile(ks, 10)),
            "p90": float(np.percentile(ks, 90))}


def settle(launch, ms):
    """Clock settle: the same launch back to back for at least `ms` of wall
    time (synchronising every 10 launches), before any counted warmup.  The
    first ~10 ms of work on an idle GPU run ~30% slower while its clocks ramp
    up.  Returns (wall ms spent, launches)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(10):
            launch()
        n += 10
        torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3, n


def time_launches(launch, steps, warmup):
    """Times `steps` back-to-back launches after `warmup` untimed ones, with
    device synchronisation around the timed region and one pair of events
    around it on the current stream (the stream the kernels are enqueued on).
    A second pass of `steps` launches with an event pair around each gives
    the spread of single launches.  Returns (wall ms per step, mean kernel us
    over the timed region, median / p10 / p90 single-launch us)."""
    import torch
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        launch()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    region_us = e0.elapsed_time(e1) * 1e3 / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        launch()
        b.record()
    torch.cuda.synchronize()
    ks = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return wall, region_us, {"median": float(np.median(ks)), "p10": float(np.percentile(ks, 10)),
                             "p90": float(np.percentile(ks, 90))}


def linear_case(wl, b, steps, warmup, x=None, rows=0, flush_reps=0, settle_ms=0.0):
    import torch
    from test_rnn_layers_head_amd import ttt_linear_fwd
    from test_rnn_layers_head_amd import inputs
    x = x or inputs.make_inputs(wl)
    d = device_inputs(x)
    z = torch.empty((wl.B, wl.H, wl.T, wl.d), device="cuda")
    w = torch.empty((wl.B, wl.H, wl.d, wl.d), device="cuda")
    launch = lambda: ttt_linear_fwd(d["q"], d["k"], d["v"], d["eta"], d["w0"], b, z=z, w_out=w,
                                    rows_per_workgroup=rows)
    settled = settle(launch, settle_ms) if settle_ms > 0 else (0.0, 0)
    wall, kmean, spread = time_launches(launch, steps, warmup)
    flushed = flushed_launches(launch, flush_reps) if flush_reps else None
    assert torch.isfinite(z).all().item()
    byts = linear_alg_bytes(wl)
    res = {
        "workload": wl.name, "b": b, "token_heads_per_s": wl.token_heads / (wall * 1e-3),
        "ms_per_step": wall, "kernel_us_mean": kmean, "kernel_us_median": spread["median"],
        "kernel_us_p10": spread["p10"], "kernel_us_p90": spread["p90"],
        "settle_ms": settled[0], "settle_launches": settled[1],
        "alg_bytes": byts, "hbm_GBps": byts / (kmean * 1e-6) / 1e9,
        "hbm_frac": byts / (kmean * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "mfma_frac": linear_alg_flops(wl, b) / (kmean * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
    }
    if flushed:
        res.update(flushed_fields(flushed, byts / 1e9 / HBM_PEAK_GBS))
    del d, z, w
    torch.cuda.empty_cache()
    return res


def flushed_fields(flushed, t_roof_s):
    """Scalar fields of a cold-cache timing (median, p10, p90 of single
    launches, each after a 512 MiB flush) and the roofline fraction of its
    median, given the kernel's roofline time in seconds."""
    return {"kernel_us_flushed_median": flushed["median"], "kernel_us_flushed_p10": flushed["p10"],
            "kernel_us_flushed_p90": flushed["p90"],
            "frac_flushed": t_roof_s / (flushed["median"] * 1e-6)}


def ln_case(wl, b, steps, warmup):
    import torch
    from test_rnn_layers_head_amd import inputs, ttt_linear_ln_fwd
    x = inputs.make_inputs(wl)
    d = device_inputs(x)
    gam = torch.from_numpy(x.ln_gamma).cuda()
    bet = torch.from_numpy(x.ln_beta).cuda()
    z = torch.empty((wl.B, wl.H, wl.T, wl.d), device="cuda")
    w = torch.empty((wl.B, wl.H, wl.d, wl.d), device="cuda")
    launch = lambda: ttt_linear_ln_fwd(d["q"], d["k"], d["v"], d["eta"], d["w0"], gam, bet,
                                       wl.ln_eps, b, z=z, w_out=w)
    wall, kmean, spread = time_launches(launch, steps, warmup)
    assert torch.isfinite(z).all().item()
    byts = ln_alg_bytes(wl)
    res = {
        "workload": wl.name, "b": b, "token_heads_per_s": wl.token_heads / (wall * 1e-3),
        "ms_per_step": wall, "kernel_us_mean": kmean, "kernel_us_median": spread["median"],
        "kernel_us_p10": spread["p10"], "kernel_us_p90": spread["p90"],
        "alg_bytes": byts, "hbm_GBps": byts / (kmean * 1e-6) / 1e9,
        "hbm_frac": byts / (kmean * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "kernel": "linear_ln_scan_kernel (one workgroup per (batch, head))",
        "traffic": traffic_for("linear_ln_scan", LN_SOURCES, wl.name),
        "sq": sq_for("linear_ln_scan", LN_SOURCES),
    }
    del d, z, w
    torch.cuda.empty_cache()
    return res


def mlp_case(wl, b, steps, warmup, flush_reps=0):
    import torch
    from test_rnn_layers_head_amd import inputs, ttt_mlp_fwd
    x = inputs.make_inputs(wl)
    d = device_inputs(x)
    z = torch.empty((wl.B, wl.H, wl.T, wl.d), device="cuda")
    w1 = torch.empty((wl.B, wl.H, wl.hidden, wl.d), device="cuda")
    w2 = torch.empty((wl.B, wl.H, wl.d, wl.hidden), device="cuda")
    launch = lambda: ttt_mlp_fwd(d["q"], d["k"], d["v"], d["eta"], d["w1"], d["w2"], b, z=z,
                                 w1_out=w1, w2_out=w2)
    wall, kmean, spread = time_launches(launch, steps, warmup)
    flushed = flushed_launches(launch, flush_reps) if flush_reps else None
    assert torch.isfinite(z).all().item()
    kmed = spread["median"]
    byts = mlp_alg_bytes(wl)
    flops = mlp_alg_flops(wl, b)
    # the kernel keeps both layers resident on chip: its roofline is the
    # algorithmic one, max(alg. bytes / HBM peak, alg. FLOPs / bf16 MFMA peak)
    t_roof = max(byts / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12))
    # secondary reading only: a design that reads and writes the 2 x hidden x
    # d fp32 state once per mini-batch (which this kernel does not do) would
    # move these bytes
    designed = byts + wl.units * ((wl.T + b - 1) // b) * 2 * (2 * wl.hidden * wl.d * 4)
    t = kmean * 1e-6
    res = {
        "workload": wl.name, "b": b, "token_heads_per_s": wl.token_heads / (wall * 1e-3),
        "ms_per_step": wall, "kernel_us_mean": kmean, "kernel_us_median": kmed,
        "kernel_us_p10": spread["p10"], "kernel_us_p90": spread["p90"],
        "alg_bytes": byts, "alg_flops": flops,
        "roofline_bound": "mfma (algorithmic)" if t_roof > byts / (HBM_PEAK_GBS * 1e9) else "hbm",
        "roofline_us": t_roof * 1e6, "roofline_frac": t_roof / t,
        "mfma_frac_algorithmic": flops / t / 1e12 / BF16_PEAK_TFLOPS,
        "hbm_frac_algorithmic": byts / t / 1e9 / HBM_PEAK_GBS,
        "secondary_state_roundtrip_hbm_frac": designed / t / 1e9 / HBM_PEAK_GBS,
        "kernel": ("mlp_primal_kernel" if wl.qkv_dtype != "bf16" or (b > 16 and b % 16)
                   else "mlp_scan_kernel" + (" (gradient point held across tiles)" if b > 16 else "")),
        # the counter summaries cover the b = 16 kernel only
        **({"traffic": traffic_for("mlp_scan", MLP_SOURCES, wl.name),
            "sq": sq_for("mlp_scan", MLP_SOURCES)} if b == 16 else {}),
    }
    if flushed:
        res.update(flushed_fields(flushed, t_roof))
    del d, z, w1, w2
    torch.cuda.empty_cache()
    return res


# Decode steps: one token for every (batch, head) unit per call, the states
# resident in HBM.  Shapes: the 1.3B layer (H = 32) and the 125M one
# (H = 12, TTT-MLP) at a serving batch of 64 sequences, b = 16, each sequence
# at its own (seeded) position in [0, 8192).
DECODE_CASES = (("linear", 64, 32), ("linear_ln", 64, 32), ("mlp", 64, 12))


def decode_alg_bytes(kind, B, H, pos, b) -> int:
    """State traffic of one step: read W, write W, and read the gradient
    point (or write it, at the first token of a mini-batch); plus the
    token's q, k, v (bf16), eta, pos and z."""
    st = 4 * 64 * 64 if kind != "mlp" else 2 * 4 * 256 * 64
    per_unit = 3 * st + 3 * 64 * 2 + 4 + 64 * 4
    extra = 2 * H * 64 * 4 if kind == "linear_ln" else 0
    return B * H * per_unit + B * 4 + extra


def decode_case(kind, B, H, steps, warmup, b=16, seed=11):
    import torch
    from test_rnn_layers_head_amd import ttt_linear_ln_step, ttt_linear_step, ttt_mlp_step
    g = torch.Generator().manual_seed(seed)
    bf = lambda *shape: (torch.randn(*shape, generator=g) / 8).to(torch.bfloat16).cuda()
    q, k, v = bf(B, H, 64), bf(B, H, 64), bf(B, H, 64)
    eta = (0.02 * torch.sigmoid(torch.randn(B, H, generator=g))).cuda()
    pos = torch.randint(0, 8192, (B,), generator=g, dtype=torch.int32).cuda()
    z = torch.empty(B, H, 64, device="cuda")
    if kind == "mlp":
        w1 = (torch.randn(B, H, 256, 64, generator=g) * 0.02).cuda()
        w2 = (torch.randn(B, H, 64, 256, generator=g) * 0.02).cuda()
        w1g, w2g = w1.clone(), w2.clone()
        launch = lambda: ttt_mlp_step(q, k, v, eta, w1, w2, w1g, w2g, pos, b, z=z)
    else:
        w = (torch.randn(B, H, 64, 64, generator=g) / 8).cuda()
        wg = w.clone()
        if kind == "linear":
            launch = lambda: ttt_linear_step(q, k, v, eta, w, wg, pos, b, z=z)
        else:
            gam = (1 + 0.2 * torch.randn(H, 64, generator=g)).cuda()
            bet = (0.1 * torch.randn(H, 64, generator=g)).cuda()
            launch = lambda: ttt_linear_ln_step(q, k, v, eta, w, wg, pos, gam, bet, 1e-5, b, z=z)
    # One launch is a few microseconds of GPU work, less than the host needs
    # to issue it from Python, so the steps are timed as a captured graph of
    # GRAPH_STEPS launches (the C ABI enqueues on the capturing stream).
    GRAPH_STEPS = 20
    for _ in range(3):
        launch()  # first launches outside the capture (code load)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(GRAPH_STEPS):
            launch()
    one = torch.cuda.CUDAGraph()
    with torch.cuda.graph(one):
        launch()
    for _ in range(max(1, warmup // GRAPH_STEPS)):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // GRAPH_STEPS)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    kmean = e0.elapsed_time(e1) * 1e3 / (reps * GRAPH_STEPS)
    # cold: one step after a 512 MiB write that evicts the MALL and the L2s
    flushed = flushed_launches(one.replay, 10)
    assert torch.isfinite(z).all().item()
    byts = decode_alg_bytes(kind, B, H, pos, b)
    return {"kind": kind, "B": B, "H": H, "b": b, "us_per_step": kmean,
            "us_per_step_flushed": flushed, "tokens_per_s": B / (kmean * 1e-6),
            "token_heads_per_s": B * H / (kmean * 1e-6), "alg_bytes": byts,
            "hbm_GBps": byts / (kmean * 1e-6) / 1e9,
            "hbm_frac": byts / (kmean * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "hbm_frac_flushed": byts / (flushed["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "timing": f"graph of {GRAPH_STEPS} steps replayed {reps} times (states resident "
                      "in HBM, and in the 256 MB MALL when they fit); flushed: single steps "
                      "after a 512 MiB cache flush"}


def bwd_alg_bytes(wl, b=16) -> int:
    """Backward with one state checkpoint per b-token mini-batch: read q, k,
    v (bf16), eta, dz and the checkpoints (64 x 64 fp32 per mini-batch);
    write dq, dk, dv, deta (fp32) and dW0."""
    per_tok = 3 * wl.d * 2 + 4 + wl.d * 4 + 3 * wl.d * 4 + 4
    nmb = (wl.T + b - 1) // b
    return wl.token_heads * per_tok + wl.units * (nmb + 1) * wl.d * wl.d * 4


def training_case(wl, steps, warmup, b=16):
    """ttt_linear_fwd_ckpt then ttt_linear_bwd on one workload, timed
    separately; dz is a seeded N(0, 0.01) draw.  Where both take sequence
    chunks, the single-pass backward is timed beside them.  bf16 with b = 16
    runs the dual-form kernels, with b < 16 the same kernels with one
    mini-batch per zero-padded tile, with b > 16 the dual-form forward and
    the primal-form backward; fp32 inputs the primal-form kernels."""
    import torch
    from test_rnn_layers_head_amd import (inputs, ttt_linear_bwd, ttt_linear_fwd_ckpt,
                                          ttt_linear_fwd_plan)
    x = inputs.make_inputs(wl)
    d = device_inputs(x)
    g = torch.Generator().manual_seed(17)
    dz = (torch.randn(wl.B, wl.H, wl.T, wl.d, generator=g) * 0.1).cuda()
    nt = (wl.T + b - 1) // b
    z = torch.empty((wl.B, wl.H, wl.T, wl.d), device="cuda")
    w = torch.empty((wl.B, wl.H, wl.d, wl.d), device="cuda")
    ck = torch.empty((wl.B, wl.H, nt, wl.d, wl.d), device="cuda")
    fwd = lambda: ttt_linear_fwd_ckpt(d["q"], d["k"], d["v"], d["eta"], d["w0"], b, z=z, w_out=w,
                                      w_ckpt=ck)
    fwd()
    bwd = lambda: ttt_linear_bwd(d["q"], d["k"], d["v"], d["eta"], ck, b, dz)
    _, kf, _ = time_launches(fwd, steps, warmup)
    _, kb, _ = time_launches(bwd, steps, warmup)
    grads = bwd()
    torch.cuda.synchronize()
    assert all(torch.isfinite(t).all().item() for t in grads)
    fb = linear_alg_bytes(wl) + wl.units * nt * wl.d * wl.d * 4
    bb = bwd_alg_bytes(wl, b)
    chunks = ttt_linear_fwd_plan(wl.B, wl.H, wl.T, b)[1]
    extra = {"seq_chunks": chunks}
    if wl.qkv_dtype != "bf16":
        extra["kernels"] = "linear_primal_ckpt_kernel / linear_primal_bwd_kernel"
    elif b > 16:
        extra["kernels"] = ("linear_scan_bf16_kernel with checkpoint stores / linear_bwd_kernel<true> "
                            "(gradient point held across b / 16 tiles)")
    else:
        extra["kernels"] = ("linear_scan_bf16_kernel with checkpoint stores / linear_bwd_kernel"
                            + (" (one mini-batch per zero-padded tile)" if b < 16 else ""))
    if chunks > 1:
        _, k1, _ = time_launches(lambda: ttt_linear_bwd(d["q"], d["k"], d["v"], d["eta"], ck, 16, dz,
                                                        seq_chunks=1), steps, warmup)
        extra["bwd_one_pass_us"] = k1
    return {"workload": wl.name, "b": b, **extra, "fwd_ckpt_us": kf, "bwd_us": kb,
            "fwd_alg_bytes": fb, "bwd_alg_bytes": bb,
            "fwd_hbm_frac": fb / (kf * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "bwd_hbm_frac": bb / (kb * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "train_token_heads_per_s": wl.token_heads / ((kf + kb) * 1e-6)}


def mlp_training_case(wl, b, steps, warmup):
    """ttt_mlp_fwd_ckpt then ttt_mlp_bwd on one TTT-MLP workload, timed
    separately; dz is a seeded N(0, 0.01) draw.  bf16 inputs: the forward is
    the dual-form scan with checkpoint stores, the backward the dual-form
    backward for b | 16 (b < 16: one mini-batch per zero-padded tile) and the
    primal form (fp32 arithmetic, one token at a time) otherwise."""
    import torch
    from test_rnn_layers_head_amd import inputs, ttt_mlp_bwd, ttt_mlp_fwd_ckpt
    x = inputs.make_inputs(wl)
    d = device_inputs(x)
    g = torch.Generator().manual_seed(19)
    dz = (torch.randn(wl.B, wl.H, wl.T, wl.d, generator=g) * 0.1).cuda()
    fwd = lambda: ttt_mlp_fwd_ckpt(d["q"], d["k"], d["v"], d["eta"], d["w1"], d["w2"], b)
    _, _, _, c1, c2 = fwd()
    bwd = lambda: ttt_mlp_bwd(d["q"], d["k"], d["v"], d["eta"], c1, c2, b, dz)
    _, kf, _ = time_launches(fwd, steps, warmup)
    _, kb, _ = time_launches(bwd, steps, warmup)
    grads = bwd()
    torch.cuda.synchronize()
    assert all(torch.isfinite(t).all().item() for t in grads)
    nmb = (wl.T + b - 1) // b
    st = 2 * wl.hidden * wl.d * 4
    fb = mlp_alg_bytes(wl) + wl.units * nmb * st
    bb = mlp_bwd_alg_bytes(wl, b)
    dual_bwd = wl.qkv_dtype == "bf16" and 16 % b == 0
    return {"workload": wl.name, "b": b, "fwd_ckpt_us": kf, "bwd_us": kb,
            "fwd_alg_bytes": fb, "bwd_alg_bytes": bb,
            "fwd_hbm_frac": fb / (kf * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "bwd_hbm_frac": bb / (kb * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "train_token_heads_per_s": wl.token_heads / ((kf + kb) * 1e-6),
            **({"bwd_traffic": traffic_for("mlp_bwd", MLP_BWD_SOURCES, wl.name),
                "bwd_sq": sq_for("mlp_bwd", MLP_BWD_SOURCES)} if dual_bwd and b == 16 else {}),
            "kernels": ("mlp_scan_kernel with checkpoint stores" if wl.qkv_dtype == "bf16" and
                        (16 % b == 0 or b % 16 == 0) else "mlp_primal_kernel (checkpoints)")
                       + (" / mlp_bwd_kernel (dual form" + (", one mini-batch per zero-padded tile)"
                                                             if b < 16 else ")")
                          if dual_bwd else " / mlp_primal_bwd_kernel")}


def ln_training_case(wl, b, steps, warmup):
    """ttt_linear_ln_fwd_ckpt then ttt_linear_ln_bwd on one LayerNorm
    workload, timed separately; dz is a seeded N(0, 0.01) draw.  bf16 with
    16 | b: the forward is the dual-form scan with checkpoint stores; bf16
    with b = 16: the backward is the dual form (four waves per unit), else the
    primal form (fp32 arithmetic, one token at a time)."""
    import torch
    from test_rnn_layers_head_amd import inputs, ttt_linear_ln_bwd, ttt_linear_ln_fwd_ckpt
    x = inputs.make_inputs(wl)
    d = device_inputs(x)
    gam = torch.from_numpy(x.ln_gamma).cuda()
    bet = torch.from_numpy(x.ln_beta).cuda()
    g = torch.Generator().manual_seed(23)
    dz = (torch.randn(wl.B, wl.H, wl.T, wl.d, generator=g) * 0.1).cuda()
    fwd = lambda: ttt_linear_ln_fwd_ckpt(d["q"], d["k"], d["v"], d["eta"], d["w0"], gam, bet,
                                         wl.ln_eps, b)
    _, _, ck = fwd()
    bwd = lambda: ttt_linear_ln_bwd(d["q"], d["k"], d["v"], d["eta"], ck, gam, bet, wl.ln_eps, b, dz)
    _, kf, _ = time_launches(fwd, steps, warmup)
    _, kb, _ = time_launches(bwd, steps, warmup)
    grads = bwd()
    torch.cuda.synchronize()
    assert all(torch.isfinite(t).all().item() for t in grads)
    nmb = (wl.T + b - 1) // b
    fb = ln_alg_bytes(wl) + wl.units * nmb * wl.d * wl.d * 4
    bb = ln_bwd_alg_bytes(wl, b)
    dual_bwd = wl.qkv_dtype == "bf16" and b == 16
    return {"workload": wl.name, "b": b, "fwd_ckpt_us": kf, "bwd_us": kb,
            "fwd_alg_bytes": fb, "bwd_alg_bytes": bb,
            "fwd_hbm_frac": fb / (kf * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "bwd_hbm_frac": bb / (kb * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "train_token_heads_per_s": wl.token_heads / ((kf + kb) * 1e-6),
            **({"bwd_traffic": traffic_for("linear_ln_bwd", LN_BWD_SOURCES, wl.name),
                "bwd_sq": sq_for("linear_ln_bwd", LN_BWD_SOURCES)} if dual_bwd else {}),
            "kernels": ("linear_ln_scan_kernel with checkpoint stores" if wl.qkv_dtype == "bf16" and b % 16 == 0
                        else "linear_ln_primal_kernel (checkpoints)")
                       + (" / linear_ln_bwd_kernel (dual form)" if wl.qkv_dtype == "bf16" and b == 16
                          else " / linear_ln_primal_bwd_kernel")}


def mlp_ln_case(wl, b, steps, warmup):
    """ttt_mlp_ln_fwd (TTT-MLP with the LayerNorm + residual wrapper) on one
    workload: the dual-form scan for bf16 inputs with b | 16 or 16 | b (the
    gradient point held across tiles for b > 16), else the primal-form
    kernel."""
    import torch
    from test_rnn_layers_head_amd import inputs, ttt_mlp_ln_fwd
    x = inputs.make_inputs(wl)
    d = device_inputs(x)
    gam = torch.from_numpy(x.ln_gamma).cuda()
    bet = torch.from_numpy(x.ln_beta).cuda()
    launch = lambda: ttt_mlp_ln_fwd(d["q"], d["k"], d["v"], d["eta"], d["w1"], d["w2"], gam, bet,
                                    wl.ln_eps, b)
    wall, kmean, spread = time_launches(launch, steps, warmup)
    byts = mlp_ln_alg_bytes(wl)
    flops = mlp_alg_flops(wl, b)
    dual = wl.qkv_dtype == "bf16" and (16 % b == 0 or b % 16 == 0)
    return {"workload": wl.name, "b": b, "token_heads_per_s": wl.token_heads / (wall * 1e-3),
            "kernel_us_mean": kmean, "kernel_us_median": spread["median"],
            "alg_bytes": byts, "alg_flops": flops,
            "hbm_frac_algorithmic": byts / (kmean * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "mfma_frac_algorithmic": flops / (kmean * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
            **({"traffic": traffic_for("mlp_ln_scan", MLP_SOURCES, wl.name),
                "sq": sq_for("mlp_ln_scan", MLP_SOURCES)} if dual and b == 16 else {}),
            "kernel": ("mlp_scan_kernel with the LayerNorm wrapper (dual form)"
                       if dual else
                       "mlp_primal_kernel with the LayerNorm wrapper (fp32, one token at a time)")}


def gate_alg_bytes(wl) -> int:
    """Learning-rate gate: read x (bf16) and theta_lr (fp32), write eta."""
    return wl.B * wl.T * wl.gate_dx * 2 + wl.H * wl.gate_dx * 4 + wl.token_heads * 4


def time_graph(launch, steps, warmup, n=20):
    """Mean GPU time per launch of `launch` captured n times in a HIP graph
    and replayed: for kernels shorter than the host's issue time per call."""
    import torch
    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(n):
            launch()
    for _ in range(max(1, warmup // n)):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // n)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * n)


def gate_case(wl, steps, warmup):
    """ttt_lr_gate alone (both launch shapes), its backward ttt_lr_gate_bwd,
    and ttt_linear_gated_fwd (gate + scan) on one gated workload."""
    import torch
    from test_rnn_layers_head_amd import inputs, ttt_linear_gated_fwd, ttt_lr_gate, ttt_lr_gate_bwd
    x = inputs.make_inputs(wl)
    d = device_inputs(x)
    gx = torch.from_numpy(x.gate_x_raw.view(np.int16)).cuda().view(torch.bfloat16)
    th = torch.from_numpy(x.theta_lr).cuda()
    eta = torch.empty((wl.B, wl.H, wl.T), device="cuda")
    z = torch.empty((wl.B, wl.H, wl.T, wl.d), device="cuda")
    w = torch.empty((wl.B, wl.H, wl.d, wl.d), device="cuda")
    gb = gate_alg_bytes(wl)
    res = {"workload": wl.name, "dx": wl.gate_dx, "gate_alg_bytes": gb}
    for tpw in (32, 64):
        _, k, spread = time_launches(lambda: ttt_lr_gate(gx, th, x.eta_base, eta=eta,
                                                         tokens_per_workgroup=tpw), steps, warmup)
        res[f"gate_us_tpw{tpw}"] = k
        res[f"gate_hbm_frac_tpw{tpw}"] = gb / (k * 1e-6) / 1e9 / HBM_PEAK_GBS
    # the same launches (automatic shape) replayed from a graph: at 125M one
    # gate launch is shorter than the host's issue time from Python
    k = time_graph(lambda: ttt_lr_gate(gx, th, x.eta_base, eta=eta), steps, warmup)
    res["gate_us_graph"] = k
    res["gate_hbm_frac_graph"] = gb / (k * 1e-6) / 1e9 / HBM_PEAK_GBS
    # backward of the gate: read x, theta, eta, deta; write dtheta, dx
    deta = torch.randn((wl.B, wl.H, wl.T), device="cuda")
    dth = torch.empty((wl.H, wl.gate_dx), device="cuda")
    dxo = torch.empty((wl.B, wl.T, wl.gate_dx), device="cuda")
    ttt_lr_gate(gx, th, x.eta_base, eta=eta)
    _, k, _ = time_launches(lambda: ttt_lr_gate_bwd(gx, th, x.eta_base, eta, deta, dtheta_lr=dth,
                                                    dx=dxo), steps, warmup)
    bb = wl.B * wl.T * wl.gate_dx * 6 + wl.H * wl.gate_dx * 8 + wl.token_heads * 8
    res["gate_bwd_us"] = k
    res["gate_bwd_alg_bytes"] = bb
    res["gate_bwd_hbm_frac"] = bb / (k * 1e-6) / 1e9 / HBM_PEAK_GBS
    k = time_graph(lambda: ttt_lr_gate_bwd(gx, th, x.eta_base, eta, deta, dtheta_lr=dth, dx=dxo),
                   steps, warmup)
    res["gate_bwd_us_graph"] = k
    res["gate_bwd_hbm_frac_graph"] = bb / (k * 1e-6) / 1e9 / HBM_PEAK_GBS
    del deta, dth, dxo
    launch = lambda: ttt_linear_gated_fwd(d["q"], d["k"], d["v"], gx, th, x.eta_base, d["w0"], 16,
                                          eta=eta, z=z, w_out=w)
    wall, k, _ = time_launches(launch, steps, warmup)
    assert torch.isfinite(z).all().item()
    res["gated_fwd_us"] = k
    res["gated_fwd_token_heads_per_s"] = wl.token_heads / (k * 1e-6)
    res["gated_fwd_alg_bytes"] = gb + linear_alg_bytes(wl)
    res["gated_fwd_hbm_frac"] = res["gated_fwd_alg_bytes"] / (k * 1e-6) / 1e9 / HBM_PEAK_GBS
    del d, gx, z, w
    torch.cuda.empty_cache()
    return res


def stream_copy_GBps(nbytes=1 << 30, reps=10):
    import torch
    from test_rnn_layers_head_amd import bench_copy
    src = torch.empty(nbytes // 4, device="cuda")
    src.fill_(1.0)
    dst = torch.empty_like(src)
    launch = lambda: bench_copy(src, dst)
    _, kmean, _ = time_launches(launch, reps, 2)
    return 2 * nbytes / (kmean * 1e-6) / 1e9


def cpu_baseline(x, b, min_seconds=3.0, nthreads=None):
    """The fp64 primal oracle as it stands, on the host cores: whole calls on
    the workload, repeated until `min_seconds` of wall time have passed."""
    from oracle import oracle
    n = nthreads or oracle.default_threads()
    q, k, v, eta = (a.astype(np.float64) for a in (x.q, x.k, x.v, x.eta))
    calls = 0
    t0 = time.perf_counter()
    while True:
        oracle.linear(q, k, v, eta, x.w0, b, nthreads=n)
        calls += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    visible = oracle.host_cores()
    return {"value": calls * x.wl.token_heads / dt, "unit": UNIT, "cores": n, "kind": "oracle",
            "host_cores_visible": visible,
            "sample": f"all {x.wl.units} (batch, head) units of {x.wl.name}, b={b}, "
                      f"fp64 sequential primal form, {calls} calls in {dt:.2f} s wall, "
                      f"{n} threads ({visible} cores visible to the process; a GPU's share of "
                      "the host is 16 cores)"}


def auto_rows(units: int) -> int:
    """Rows of W per workgroup that the library picks for `units` (batch,
    head) units when the caller passes 0."""
    return 64 if units >= 256 else (32 if units > 64 else 16)


def traffic_for(kernel_key: str, sources, workload: str):
    """HBM bytes per launch from committed counter readings (FETCH_SIZE +
    WRITE_SIZE, scaled by the copy-kernel calibration), or None if the
    readings are missing, were taken on different kernel sources, or on
    another workload."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    e = t.get(kernel_key)
    if not e or e.get("source_hash") != source_hash(sources) or e.get("workload") != workload:
        return None
    return e["bytes_per_launch"]


# --------------------------------------------------------------------------
# Counter summary: rocprofv3 --pmc output -> profiles/traffic_counters.json
# --------------------------------------------------------------------------
def summarize_pmc(fetch_dir, write_dir):
    """Reads one FETCH_SIZE and one WRITE_SIZE rocprofv3 run of
    `bench.py --no-extras --no-cpu --pmc-calibrate`, scales both counters by
    what they read for the 1 GiB streaming copy, writes the per-launch HBM
    bytes of each scan kernel to profiles/traffic_counters.json and prints a
    report (per-dispatch readings, calibration, ratio to algorithmic bytes)."""
    import csv
    from test_rnn_layers_head_amd import inputs

    def read(dirname, counter):
        agg = {}
        for path in glob.glob(os.path.join(dirname, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") == counter:  # sum over hardware instances
                        key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
                        agg[key] = agg.get(key, 0.0) + float(r["Counter_Value"])
        return agg

    raw = {"FETCH_SIZE": read(fetch_dir, "FETCH_SIZE"), "WRITE_SIZE": read(write_dir, "WRITE_SIZE")}
    med = {}
    for c, agg in raw.items():
        per = {}
        for (_, name), val in agg.items():
            per.setdefault(name, []).append(val)
        med[c] = {k: float(np.median(v)) for k, v in per.items()}
    fetch, write = med["FETCH_SIZE"], med["WRITE_SIZE"]
    copy_name = next(k for k in fetch if "stream_copy_kernel" in k)
    copy_bytes = 1 << 30  # --pmc-calibrate copies 1 GiB
    f_scale = copy_bytes / (fetch[copy_name] * 1024.0)
    w_scale = copy_bytes / (write[copy_name] * 1024.0)
    out = {"calibration": {"copy_bytes": copy_bytes, "fetch_kib": fetch[copy_name],
                           "write_kib": write[copy_name], "fetch_scale": f_scale,
                           "write_scale": w_scale}}
    print("Per-dispatch readings of the scan and calibration kernels (KiB, summed over instances):")
    for c, agg in raw.items():
        for (disp, name), val in sorted(agg.items()):
            if "scan" in name or "stream_copy" in name:
                print(f"  {c:10s} dispatch {disp:>3d}  {val:14.3f}  {name[:60]}")
    print(f"\nCalibration: stream_copy_kernel over 1 GiB reads {fetch[copy_name]:.0f} KiB by "
          f"FETCH_SIZE and writes {write[copy_name]:.0f} KiB by WRITE_SIZE;\nscale factors fetch "
          f"x{f_scale:.4f}, write x{w_scale:.4f} (each factor: the bytes the copy moves over what the "
          "counter reads for it).\n")
    cases = (("linear_scan", "linear_scan_bf16_kernel", SCAN_SOURCES, linear_alg_bytes, 3),
             ("linear_ln_scan", LN_SCAN_NAME, LN_SOURCES, ln_alg_bytes, 6),
             ("mlp_scan", MLP_SCAN_NAME, MLP_SOURCES, mlp_alg_bytes, 4),
             ("mlp_ln_scan", MLP_LN_SCAN_NAME, MLP_SOURCES, mlp_ln_alg_bytes, 10),
             ("mlp_bwd", "mlp_bwd_kernel", MLP_BWD_SOURCES, mlp_bwd_alg_bytes, 4),
             ("linear_ln_bwd", "linear_ln_bwd_kernel", LN_BWD_SOURCES, ln_bwd_alg_bytes, 7))
    for key, pat, srcs, alg_fn, wid in cases:
        names = [k for k in fetch if pat in k]
        if not names:
            continue
        n = names[0]
        byts = fetch[n] * 1024 * f_scale + write.get(n, 0.0) * 1024 * w_scale
        wl = inputs.workload(wid)
        alg = alg_fn(wl)
        out[key] = {"kernel": n, "workload": wl.name, "fetch_kib": fetch[n],
                    "write_kib": write.get(n, 0.0), "bytes_per_launch": byts,
                    "alg_bytes_per_launch": alg, "source_hash": source_hash(srcs)}
        print(f"{key}: {n}\n  workload {wl.name}: median FETCH {fetch[n]:.1f} KiB, WRITE "
              f"{write.get(n, 0.0):.1f} KiB -> {byts / 1e6:.1f} MB per launch (scaled)\n"
              f"  algorithmic bytes per launch {alg / 1e6:.1f} MB -> measured/algorithmic = "
              f"{byts / alg:.3f}\n  kernel source hash {source_hash(srcs)}")
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)


# --------------------------------------------------------------------------
# SQ counter summary: rocprofv3 --pmc (MFMA / VALU activity) -> JSON + text
# --------------------------------------------------------------------------
SQ_FILE = os.path.join(ROOT, "profiles", "sq_counters.json")
SQ_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
               "SQ_ACTIVE_INST_VALU", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY")
SIMDS, CUS, XCDS = 1024, 256, 8  # MI355X: 8 XCDs x 32 CUs x 4 SIMDs


def sq_derive(med, active_cus):
    """Per-kernel readings from the dispatch's counter values (rocprofv3
    reports each counter summed over its hardware instances):
      clock      = GRBM_GUI_ACTIVE / XCDs: the kernel's duration in GPU
                   cycles (the counter runs once per XCD);
      mfma_busy  = SQ_VALU_MFMA_BUSY_CYCLES / (clock * SIMDs): the fraction
                   of the chip's SIMD-cycles the matrix unit is busy (the
                   counter sums busy cycles over SIMDs; one 16x16x32 bf16
                   MFMA reads 16);
      valu_busy  = 4 SQ_ACTIVE_INST_VALU / (clock * SIMDs): the same for VALU
                   issue (the counter is in quad-cycles: one per wave64 VALU
                   instruction, as SQ_INSTS_VALU shows);
      *_active   = the same over the SIMDs of the CUs that have work
                   (one workgroup per CU: min(workgroups, CUs));
      wait_frac  = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (wave-cycles waiting)."""
    clock = med["GRBM_GUI_ACTIVE"] / XCDS
    mfma = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (clock * SIMDS)
    valu = 4.0 * med["SQ_ACTIVE_INST_VALU"] / (clock * SIMDS)
    share = CUS / active_cus
    return {"clock_cycles": clock, "mfma_busy": mfma, "valu_busy": valu,
            "mfma_busy_active": mfma * share, "valu_busy_active": valu * share,
            "mfma_cycles_per_inst": med["SQ_VALU_MFMA_BUSY_CYCLES"] / med["SQ_INSTS_MFMA"],
            "wait_frac": med["SQ_WAIT_INST_ANY"] / med["SQ_WAVE_CYCLES"]}


SQ_CASES = (("linear_scan", "linear_scan_bf16_kernel", "SCAN_SOURCES", 256),   # 2 workgroups x 128 units
            ("linear_ln_scan", LN_SCAN_NAME, "LN_SOURCES", 128),   # 128 units
            ("mlp_scan", MLP_SCAN_NAME, "MLP_SOURCES", 96),                     # 96 units
            ("mlp_ln_scan", MLP_LN_SCAN_NAME, "MLP_SOURCES", 96),
            ("mlp_bwd", "mlp_bwd_kernel", "MLP_BWD_SOURCES", 96),
            ("linear_ln_bwd", "linear_ln_bwd_kernel", "LN_BWD_SOURCES", 96))


def summarize_sq(sq_dir):
    """Reads one rocprofv3 --pmc run of `bench.py --no-extras --no-cpu
    --pmc-calibrate` with SQ_COUNTERS and reports, per scan kernel (median
    over its dispatches), the readings of sq_derive plus instruction counts.
    Writes profiles/sq_counters.json (source-hashed per kernel, as the
    traffic counters are).  A JSON file written earlier can be given instead
    of the run's directory: the readings are then derived again from its
    medians (same sources required)."""
    import csv
    vals = {}
    meds = {}
    if sq_dir.endswith(".json"):
        with open(sq_dir) as f:
            old = json.load(f)
        meds = {k: {c: old[k][c] for c in SQ_COUNTERS} | {"dispatches": old[k]["dispatches"]}
                for k, _, _, _ in SQ_CASES if k in old}
    else:
        for path in glob.glob(os.path.join(sq_dir, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    c = r.get("Counter_Name")
                    if c in SQ_COUNTERS:
                        key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
                        d = vals.setdefault(key, {})
                        d[c] = d.get(c, 0.0) + float(r["Counter_Value"])
        for key, pat, _, _ in SQ_CASES:
            rows = [d for (disp, name), d in sorted(vals.items()) if pat in name and
                    all(c in d for c in SQ_COUNTERS)]
            if rows:
                meds[key] = {c: float(np.median([d[c] for d in rows])) for c in SQ_COUNTERS}
                meds[key]["dispatches"] = len(rows)
    out = {"counters": list(SQ_COUNTERS), "simds": SIMDS, "cus": CUS, "xcds": XCDS}
    print("SQ counters per dispatch (medians over each kernel's dispatches):")
    for key, pat, srcs, active in SQ_CASES:
        if key not in meds:
            continue
        med = meds[key]
        e = {**med, **sq_derive(med, active), "active_cus": active,
             "source_hash": source_hash(globals()[srcs])}
        out[key] = e
        print(f"{key} ({pat}, {med['dispatches']} dispatches): {e['clock_cycles']:.0f} GPU cycles; "
              f"MFMA busy {e['mfma_busy']:.3f} of all SIMD-cycles ({e['mfma_busy_active']:.3f} on the "
              f"{active} CUs with work; {e['mfma_cycles_per_inst']:.1f} cycles per MFMA), VALU busy "
              f"{e['valu_busy']:.3f} ({e['valu_busy_active']:.3f}), waves waiting "
              f"{e['wait_frac']:.3f} of wave-cycles;\n  per dispatch: {med['SQ_INSTS_MFMA']:.4g} MFMA "
              f"and {med['SQ_INSTS_VALU']:.4g} VALU instructions, source hash {e['source_hash']}")
    os.makedirs(os.path.dirname(SQ_FILE), exist_ok=True)
    with open(SQ_FILE, "w") as f:
        json.dump(out, f, indent=1)


def sq_for(kernel_key: str, sources):
    """MFMA-busy fraction from committed SQ counters, or None when missing or
    taken on other kernel sources."""
    if not os.path.exists(SQ_FILE):
        return None
    with open(SQ_FILE) as f:
        e = json.load(f).get(kernel_key)
    if not e or e.get("source_hash") != source_hash(sources):
        return None
    return {k: e[k] for k in ("mfma_busy", "valu_busy", "mfma_busy_active", "valu_busy_active",
                              "wait_frac")}


# --------------------------------------------------------------------------
# Kernel-trace summary: rocprofv3 --kernel-trace --stats output -> text
# --------------------------------------------------------------------------
def summarize_trace(trace_dir, pattern, skip, take):
    """Prints the per-kernel statistics of a rocprofv3 kernel-trace run and
    the mean duration of dispatches [skip, skip + take) of the kernels whose
    name contains `pattern` (in dispatch order; skip < 0: the last `take`).
    With skip = -1 and take = steps of a `--no-extras` run this is the timed
    region of the headline."""
    import csv
    stats = glob.glob(os.path.join(trace_dir, "**", "*_kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(trace_dir, "**", "*_kernel_trace.csv"), recursive=True)
    print("rocprofv3 kernel statistics (all dispatches of the run):")
    print(f"  {'calls':>6s} {'avg us':>10s} {'min us':>10s} {'max us':>10s}  kernel")
    for path in stats:
        for r in csv.DictReader(open(path)):
            print(f"  {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
                  f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f}  {r['Name'][:90]}")
    rows = []
    for path in trace:
        for r in csv.DictReader(open(path)):
            if pattern in r["Kernel_Name"]:
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    if skip < 0:  # the last `take` dispatches of the run
        skip = max(0, len(rows) - take)
    sel = rows[skip:skip + take]
    if sel:
        d = np.array([(e - b) / 1e3 for b, e, _ in sel])
        print(f"\ndispatches {skip} .. {skip + len(sel) - 1} of '{pattern}' ({sel[0][2][:80]}):")
        print(f"  mean {d.mean():.1f} us, median {np.median(d):.1f} us, min {d.min():.1f}, max {d.max():.1f}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed launches after the clock-settle phase")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="wall time of back-to-back headline launches before the warmup "
                         "(an idle GPU's clocks take ~0.1 s to ramp up)")
    ap.add_argument("--no-extras", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--pmc-calibrate", action="store_true",
                    help="also launch the 1 GiB streaming copy used to scale byte counters")
    ap.add_argument("--only", choices=("train", "train-long", "train-mlp", "decode", "gate"),
                    help="run one group of the secondary measurements and print it (for profiling)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-sq", metavar="SQ_DIR",
                    help="summarise a rocprofv3 --pmc run with the SQ counters (MFMA / VALU busy)")
    ap.add_argument("--summarize-trace", nargs=4, metavar=("TRACE_DIR", "KERNEL", "SKIP", "TAKE"),
                    help="summarise a rocprofv3 --kernel-trace --stats run of this script")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return 0
    if args.summarize_sq:
        summarize_sq(args.summarize_sq)
        return 0
    if args.summarize_trace:
        d, k, skip, take = args.summarize_trace
        summarize_trace(d, k, int(skip), int(take))
        return 0
    if args.gpus != 1:
        print(f"bench.py: the scan runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the scan shards over (batch, head) units with no communication)",
              file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: multi-rank launch is not supported (one GPU only)", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    from test_rnn_layers_head_amd import _lib, inputs
    _lib.lib()  # fail loudly if the HIP library is missing

    wl = inputs.workload(3)
    if args.only == "train":
        print(json.dumps({w.name: training_case(w, max(5, args.steps // 5), 10)
                          for w in (wl, inputs.workload(2))}))
        return 0
    if args.only == "train-mlp":
        w4 = inputs.workload(4)
        print(json.dumps({w4.name: mlp_training_case(w4, 16, 3, 2)}))
        return 0
    if args.only == "train-long":
        w5 = inputs.workload(5)
        print(json.dumps({w5.name: training_case(w5, 3, 2)}))
        return 0
    if args.only == "gate":
        print(json.dumps({inputs.workload(i).name: gate_case(inputs.workload(i), 20, 20)
                          for i in (8, 9)}))
        return 0
    if args.only == "decode":
        print(json.dumps({f"decode-{k}-B{B}-H{H}": decode_case(k, B, H, 100, 200)
                          for k, B, H in DECODE_CASES}))
        return 0
    b = 16
    log(f"[bench] generating {wl.name} inputs")
    x = inputs.make_inputs(wl)
    log(f"[bench] timing ttt_linear_fwd on {wl.name}: {args.settle_ms:.0f} ms clock settle, "
        f"{args.warmup} warmup + {args.steps} steps")
    head = linear_case(wl, b, args.steps, args.warmup, x=x, flush_reps=0 if args.no_extras else 20,
                       settle_ms=args.settle_ms)
    log(f"[bench] {head['kernel_us_mean']:.1f} us/launch, {head['hbm_frac']:.3f} of HBM peak")

    if args.pmc_calibrate:
        log("[bench] streaming copy calibration (1 GiB)")
        stream_copy_GBps(1 << 30, reps=3)
        w4 = inputs.workload(4)
        log(f"[bench] {w4.name} (counter coverage of the MLP scan, launches after cache flushes)")
        mlp_case(w4, 16, 2, 1, flush_reps=2)
        w6 = inputs.workload(6)
        log(f"[bench] {w6.name} (counter coverage of the LayerNorm scan)")
        ln_case(w6, 16, 2, 1)
        w10 = inputs.workload(10)
        log(f"[bench] {w10.name} (counter coverage of the MLP scan with the LayerNorm wrapper)")
        mlp_ln_case(w10, 16, 2, 1)
        log(f"[bench] {w4.name} training (counter coverage of the MLP backward)")
        mlp_training_case(w4, 16, 2, 1)
        w7 = inputs.workload(7)
        log(f"[bench] {w7.name} training (counter coverage of the LayerNorm backward)")
        ln_training_case(w7, 16, 2, 1)

    extras = {}
    if not args.no_extras:
        for bb in (1, 4, 64):
            log(f"[bench] b sweep b={bb}")
            extras[f"{wl.name}_b{bb}"] = linear_case(wl, bb, max(3, args.steps // 4), EXTRA_WARMUP,
                                                     x=x)
        for wid in (2, 5):
            w2 = inputs.workload(wid)
            log(f"[bench] {w2.name}")
            # the 125M inputs (128 MB) fit in the 256 MB MALL: also timed cold
            extras[w2.name] = linear_case(w2, 16, max(5, args.steps // 2), EXTRA_WARMUP,
                                          flush_reps=10 if wid == 2 else 0)
        for wid in (6, 7):
            w6 = inputs.workload(wid)
            log(f"[bench] {w6.name}")
            extras[w6.name] = ln_case(w6, 16, max(5, args.steps // 2), EXTRA_WARMUP)
        for wid in (8, 9):
            wg = inputs.workload(wid)
            log(f"[bench] learning-rate gate and gated scan, {wg.name}")
            extras[f"gate-{wg.name}"] = gate_case(wg, max(5, args.steps // 2), 20)
        log(f"[bench] forward with checkpoints + backward, {wl.name}")
        extras[f"train-{wl.name}"] = training_case(wl, max(5, args.steps // 5), 10)
        w5 = inputs.workload(5)
        log(f"[bench] forward with checkpoints + backward, {w5.name}")
        extras[f"train-{w5.name}"] = training_case(w5, 3, 2)
        log(f"[bench] forward with checkpoints + backward, {wl.name}, b = 4 (padded tiles)")
        extras[f"train-{wl.name}_b4"] = training_case(wl, 2, 1, b=4)
        log(f"[bench] forward with checkpoints + backward, {wl.name}, b = 64 (gradient point held)")
        extras[f"train-{wl.name}_b64"] = training_case(wl, 5, 2, b=64)
        w7 = inputs.workload(7)
        log(f"[bench] forward with checkpoints + backward, {w7.name}")
        extras[f"train-{w7.name}"] = ln_training_case(w7, 16, 2, 1)
        for kind, B, H in DECODE_CASES:
            log(f"[bench] decode step {kind} B={B} H={H}")
            extras[f"decode-{kind}-B{B}-H{H}"] = decode_case(kind, B, H, 100, 200)
        w4 = inputs.workload(4)
        log(f"[bench] {w4.name}")
        try:
            extras[w4.name] = mlp_case(w4, 16, max(5, args.steps // 2), EXTRA_WARMUP, flush_reps=10)
        except Exception as e:  # reported, never silently replaced
            extras[w4.name] = {"error": str(e)}
        log(f"[bench] {w4.name} with b = 64 (the gradient point held across four tiles)")
        extras[f"{w4.name}_b64"] = mlp_case(w4, 64, 3, 2)
        log(f"[bench] forward with checkpoints + backward, {w4.name}")
        extras[f"train-{w4.name}"] = mlp_training_case(w4, 16, 5, 2)
        w10 = inputs.workload(10)
        log(f"[bench] {w10.name} (MLP with the LayerNorm wrapper)")
        extras[w10.name] = mlp_ln_case(w10, 16, max(5, args.steps // 2), EXTRA_WARMUP)
        log("[bench] streaming copy reference")
        extras["stream_copy_GBps"] = stream_copy_GBps()
        extras["headline_frac_of_stream_copy"] = head["hbm_GBps"] / extras["stream_copy_GBps"]

    cpu = None
    if not args.no_cpu:
        log("[bench] timing the fp64 oracle on the host (CPU baseline)")
        cpu = cpu_baseline(x, b)
        if not args.no_extras:
            for wid in (1, 2):
                wx = inputs.make_inputs(inputs.workload(wid))
                log(f"[bench] fp64 oracle, one thread, {wx.wl.name}")
                extras[f"cpu_oracle_1thread_{wx.wl.name}"] = cpu_baseline(wx, 16, 1.0, nthreads=1)

    traffic = traffic_for("linear_scan", SCAN_SOURCES, wl.name)
    rec = {
        "metric": METRIC,
        "value": head["token_heads_per_s"],
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": head["settle_ms"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "inputs_sha256": x.sha256(),  # the seeded headline inputs, as both sides consume them
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "d": wl.d, "b": b,
                   "qkv_dtype": "bf16", "state_dtype": "f32", "global_batch": wl.B,
                   "seq_len": wl.T, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": head["hbm_GBps"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": head["hbm_frac"], "traffic": traffic,
                     "kernel": f"linear_scan_bf16_kernel (b=16, {auto_rows(wl.units)} rows of W per workgroup)",
                     "alg_bytes_per_launch": head["alg_bytes"],
                     "kernel_us_mean": head["kernel_us_mean"],
                     "kernel_us_median": head["kernel_us_median"],
                     "kernel_us_p10": head["kernel_us_p10"],
                     "kernel_us_p90": head["kernel_us_p90"],
                     "settle_ms": head["settle_ms"], "settle_launches": head["settle_launches"],
                     **{k: head[k] for k in ("kernel_us_flushed_median", "kernel_us_flushed_p10",
                                             "kernel_us_flushed_p90", "frac_flushed") if k in head},
                     "mfma_frac": head["mfma_frac"],
                     "mfma_busy": sq_for("linear_scan", SCAN_SOURCES)},
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
