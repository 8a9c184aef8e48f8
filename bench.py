#!/usr/bin/env python3
"""LLoPS hot-path benchmark on one MI355X.

Default: the causal forward at n=65536, p=2, t=4, m=256 (batch 1, 32 heads,
d=dv=128, bf16 inputs, fp32 accumulation/outputs, squared features,
normaliser delta=1e-6) -- one step is one full llops_linattn_causal_fwd call
(feature maps of Q and K, segment states, scan, chunked output pass) over the
whole batch, inputs resident in HBM. Prints ONE JSON line.

The line also carries:
  roofline      dominant kernel (the bf16 MFMA feature map) against the bf16
                dense MFMA peak, its duration timed live with HIP events;
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload;
  decode        the single-token decode step (batch 128, 32 heads, 1000
                consecutive steps from a 4096-token prefix state) against HBM,
                and the gated decode step over the same tokens;
  gated         the gated (decaying-state) causal pass on the same inputs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="causal_long_n65536")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads' per-config lines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gated", action="store_true", help="skip the gated causal pass")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU budget of the oracle baseline")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--power", action="store_true",
                    help="also sample the board's power (amdgpu hwmon sysfs) while the causal "
                         "step loops on each path and at idle: watts and joules per step")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (calibrates rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE against known bytes)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work (per call, whole batch)
# ---------------------------------------------------------------------------
# (m, dv) shapes of the 32x32x16 segment kernels, which walk 32-token chunks
# whatever chunk length is asked for (the chunk only orders the rounding)
_SEG32 = {(256, 128), (128, 64), (64, 64)}


def kernel_chunk(w):
    """Tokens per intra-chunk block the causal kernels actually run: 32 on
    the 32x32x16 segment kernels; the generic bf16 kernels take 32 when a
    chunk of at most 32 is asked for, else 64; the fp32 kernels take the
    requested chunk (64 by default)."""
    if w.dtype == "bf16":
        if (w.m, w.dv) in _SEG32:
            return 32
        return 32 if 0 < w.chunk <= 32 else 64
    return w.chunk if w.chunk > 0 else 64


def causal_flops(w):
    """Feature maps of Q and K, state build phi_K^T V and read-out phi_Q S, and
    the lower triangle (diagonal included) of the intra-chunk products at the
    chunk length the kernels run (kernel_chunk); normaliser and epilogue terms
    excluded."""
    bh = w.batch * w.heads
    C = kernel_chunk(w)
    per_bh = (4.0 * w.n * w.d * w.p * w.t * w.m + 4.0 * w.n * w.m * w.dv
              + w.n * (C + 1) * (w.m + w.dv))
    return bh * per_bh


def step_kernel_flops(w, kern):
    """Algorithmic flops per launch of each kernel of one causal step (whole
    batch): the feature map projects Q and K (two-kernel path) or K only
    (when the fused output pass, attn_out_fq, projects Q); the state pass
    builds phi_K^T V; an output pass reads out phi_Q S plus the intra-chunk
    triangle at the chunk it runs (its S update repeats the state pass's
    product and is not credited again)."""
    bh = w.batch * w.heads
    proj = 2.0 * w.n * w.d * w.p * w.t * w.m
    readout = 2.0 * w.n * w.m * w.dv + w.n * (kernel_chunk(w) + 1) * (w.m + w.dv)
    fused = "attn_out_fq" in kern
    table = {"featmap_bf16": bh * proj * (1 if fused else 2),
             "seg_state_bf16": bh * 2.0 * w.n * w.m * w.dv,
             "attn_out_bf16": bh * readout,
             "attn_out_fq": bh * (proj + readout)}
    return {k: v for k, v in table.items() if k in kern}


def decode_bytes(w):
    """HBM bytes one decode step must move: fp32 state S and normaliser z read
    and written, Theta_q/Theta_k read, q/k/v read (bf16), output written."""
    bh = w.batch * w.heads
    return (2 * bh * w.m * w.dv * 4 + 2 * bh * w.m * 4 + 2 * w.heads * w.p * w.t * w.d * w.m * 2
            + bh * (2 * w.d + w.dv) * 2 + bh * w.dv * 4)


def decode_state_bytes(w):
    """Bytes the decode state kernel must move per launch: S and z read and
    written, phi_q/phi_k (fp32) and v read, output written."""
    bh = w.batch * w.heads
    return 2 * bh * w.m * w.dv * 4 + 2 * bh * w.m * 4 + 2 * bh * w.m * 4 + bh * w.dv * 2 \
        + bh * w.dv * 4


# ---------------------------------------------------------------------------
def to_dev(a, torch, dtype):
    return torch.from_numpy(a).to("cuda").to(dtype)


def bench_causal(w, steps, warmup, torch, lib):
    from learnable_polynomial_feature_amd.workloads import generate
    log(f"generating {w.name} inputs")
    x = generate(w)
    g = {k: to_dev(v, torch, torch.bfloat16) for k, v in x.items()}
    del x
    out = torch.empty((w.batch, w.heads, w.n, w.dv), dtype=torch.float32, device="cuda")
    shape = lib.make_shape(batch=w.batch, heads=w.heads, n=w.n, d=w.d, dv=w.dv, m=w.m, p=w.p,
                           t=w.t, square=w.square, normalize=w.normalize, delta=w.delta,
                           chunk=w.chunk)
    ws = torch.empty(lib.llops_workspace_bytes(shape, lib.ENTRY_CAUSAL), dtype=torch.uint8,
                     device="cuda")
    args = (g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"])
    kw = dict(square=w.square, normalize=w.normalize, delta=w.delta, chunk=w.chunk, out=out,
              workspace=ws)
    log(f"warmup {warmup}")
    for _ in range(warmup):
        lib.llops_linattn_causal_fwd(*args, **kw)
    torch.cuda.synchronize()
    timer = lib.KernelTimer(capacity=16 * steps)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    log(f"timing {steps} steps")
    torch.cuda.synchronize()
    with timer:
        t0.record()
        for _ in range(steps):
            lib.llops_linattn_causal_fwd(*args, **kw)
        t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    kern = {k: sum(v) / len(v) for k, v in timer.durations_ms().items()}
    return ms, kern, (args, ws)


def bench_other_path(w, steps, torch, lib, args, ws, fused):
    """The same causal step on the other execution path: fused = True runs
    the output pass that projects phi_Q itself (LLOPS_FUSED_Q=1, phi_Q never
    in HBM); fused = False the two-kernel path (phi_Q and phi_K through HBM,
    then the segment passes)."""
    out = torch.empty((w.batch, w.heads, w.n, w.dv), dtype=torch.float32, device="cuda")
    kw = dict(square=w.square, normalize=w.normalize, delta=w.delta, chunk=w.chunk, out=out,
              workspace=ws)
    prev = os.environ.get("LLOPS_FUSED_Q")
    os.environ["LLOPS_FUSED_Q"] = "1" if fused else "0"
    try:
        for _ in range(2):
            lib.llops_linattn_causal_fwd(*args, **kw)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            lib.llops_linattn_causal_fwd(*args, **kw)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        timer = lib.KernelTimer(capacity=16 * steps)
        with timer:
            for _ in range(steps):
                lib.llops_linattn_causal_fwd(*args, **kw)
        torch.cuda.synchronize()
    finally:
        if prev is None:
            del os.environ["LLOPS_FUSED_Q"]
        else:
            os.environ["LLOPS_FUSED_Q"] = prev
    kern = {k: sum(v) / len(v) for k, v in timer.durations_ms().items()}
    del out
    kfl = step_kernel_flops(w, kern)
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(w.batch * w.n / (ms * 1e-3), 1),
            "mfma_frac_step": round(causal_flops(w) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernel_ms": {k: round(v, 4) for k, v in kern.items()},
            "kernel_mfma": {k: {"tflop_per_launch": round(f / 1e12, 4),
                                "frac": round(f / (kern[k] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
                            for k, f in kfl.items()},
            "note": ("phi_Q projected inside the output pass, never in HBM (LLOPS_FUSED_Q=1)"
                     if fused else "phi_Q and phi_K written to HBM by the feature map, read "
                                   "back by the segment passes")}


def bench_gated(w, steps, torch, lib, args, ws_causal):
    """The gated causal pass (per-token state decay exp(g), g = log sigmoid
    of N(4, 1) draws) on the same device inputs as the causal step."""
    from learnable_polynomial_feature_amd.workloads import log_gates
    del ws_causal
    lg = torch.from_numpy(log_gates(w, mu=4.0)).to("cuda")
    out = torch.empty((w.batch, w.heads, w.n, w.dv), dtype=torch.float32, device="cuda")
    shape = lib.make_shape(batch=w.batch, heads=w.heads, n=w.n, d=w.d, dv=w.dv, m=w.m, p=w.p,
                           t=w.t, square=w.square, normalize=w.normalize, delta=w.delta,
                           chunk=w.chunk)
    ws = torch.empty(lib.llops_workspace_bytes(shape, lib.ENTRY_GATED_CAUSAL), dtype=torch.uint8,
                     device="cuda")
    kw = dict(square=w.square, normalize=w.normalize, delta=w.delta, chunk=w.chunk, out=out,
              workspace=ws)
    for _ in range(2):
        lib.llops_linattn_gated_causal_fwd(*args, lg, **kw)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        lib.llops_linattn_gated_causal_fwd(*args, lg, **kw)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    timer = lib.KernelTimer(capacity=16 * steps)
    with timer:
        for _ in range(steps):
            lib.llops_linattn_gated_causal_fwd(*args, lg, **kw)
    torch.cuda.synchronize()
    kern = {k: sum(v) / len(v) for k, v in timer.durations_ms().items()}
    fl = causal_flops(w)
    del lg, out, ws
    return {"workload": f"gated causal {w.batch}x{w.heads}x{w.n} d={w.d} dv={w.dv} m={w.m} "
                        f"p={w.p} t={w.t}, squared, normalised, log gates log(sigmoid(N(4,1)))",
            "ms_per_call": round(ms, 4), "tokens_per_s": round(w.batch * w.n / (ms * 1e-3), 1),
            "mfma_frac_step": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernel_ms": {k: round(v, 4) for k, v in kern.items()}}


def attention_flops(w):
    """Algorithmic flops of one call: causal_flops for causal workloads; for
    the non-causal form the feature maps plus phi_K^T V and phi_Q S."""
    if w.causal:
        return causal_flops(w)
    bh = w.batch * w.heads
    return bh * (4.0 * w.n * w.d * w.p * w.t * w.m + 4.0 * w.n * w.m * w.dv)


def bench_config(w, steps, warmup, torch, lib):
    """One full-batch call of the workload's entry point, inputs resident in
    HBM: (ms per call, kernel ms)."""
    from learnable_polynomial_feature_amd.workloads import generate
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    x = generate(w)
    g = {k: to_dev(v, torch, dt) for k, v in x.items()}
    del x
    args = (g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"])
    kw = dict(square=w.square, normalize=w.normalize, delta=w.delta)
    out = torch.empty((w.batch, w.heads, w.n, w.dv), dtype=torch.float32, device="cuda")
    if w.causal:
        shape = lib.make_shape(batch=w.batch, heads=w.heads, n=w.n, d=w.d, dv=w.dv, m=w.m,
                               p=w.p, t=w.t, square=w.square, normalize=w.normalize,
                               delta=w.delta, chunk=w.chunk,
                               in_dtype=lib.BF16 if w.dtype == "bf16" else lib.F32)
        ws = torch.empty(lib.llops_workspace_bytes(shape, lib.ENTRY_CAUSAL), dtype=torch.uint8,
                         device="cuda")

        def call():
            lib.llops_linattn_causal_fwd(*args, chunk=w.chunk, out=out, workspace=ws, **kw)
    else:
        shape = lib.make_shape(batch=w.batch, heads=w.heads, n=w.n, d=w.d, dv=w.dv, m=w.m,
                               p=w.p, t=w.t, square=w.square, normalize=w.normalize,
                               delta=w.delta, in_dtype=lib.BF16 if w.dtype == "bf16" else lib.F32)
        ws = torch.empty(max(1, lib.llops_workspace_bytes(shape, lib.ENTRY_LINATTN)),
                         dtype=torch.uint8, device="cuda")

        def call():
            lib.llops_linattn_fwd(*args, out=out, workspace=ws, **kw)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    # calls back to back (host launch work included), then the kernels timed
    # one by one in a second pass (their events would sit between them)
    t0.record()
    for _ in range(steps):
        call()
    t1.record()
    torch.cuda.synchronize()
    eager_ms = t0.elapsed_time(t1) / steps
    timer = lib.KernelTimer(capacity=8 * steps)
    with timer:
        for _ in range(steps):
            call()
    torch.cuda.synchronize()
    kern = {k: sum(v) / len(v) for k, v in timer.durations_ms().items()}
    # one call captured as a HIP graph and replayed: no host work per call
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        call()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    graph_ms = t0.elapsed_time(t1) / steps
    del graph
    return eager_ms, kern, graph_ms


def featmap_variants(steps, torch, lib):
    """The feature map alone on the p = 4 / t = 1 and BASED-shaped variants at
    the long workload's geometry (1 x 32 heads x 65536 rows, d = 128, m = 256,
    bf16 phi), against the bf16 MFMA peak."""
    res = {}
    g = torch.Generator(device="cpu").manual_seed(5)
    B, H, n, d, m = 1, 32, 65536, 128, 256
    X = (torch.randn(B, H, n, d, generator=g) * 0.5).to(torch.bfloat16).to("cuda")
    for name, p, t in (("p4_t1", 4, 1), ("based_p2_t1", 2, 1)):
        th = (torch.randn(H, p, t, d, m, generator=g) / d ** 0.5).to(torch.bfloat16).to("cuda")
        shape = lib.make_shape(batch=B, heads=H, n=n, d=d, dv=1, m=m, p=p, t=t, square=False,
                               in_dtype=lib.BF16, out_dtype=lib.BF16)
        ws = torch.empty(max(1, lib.llops_workspace_bytes(shape, lib.ENTRY_FEATMAP)),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty((B, H, n, m), dtype=torch.bfloat16, device="cuda")

        def call():
            lib.llops_featmap(X, th, out=out, out_dtype=torch.bfloat16, workspace=ws)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        timer = lib.KernelTimer(capacity=4 * steps)
        with timer:
            for _ in range(steps):
                call()
        torch.cuda.synchronize()
        kern = {k: sum(v) / len(v) for k, v in timer.durations_ms().items()}
        fl = 2.0 * B * H * n * d * p * t * m
        ms = kern["featmap_bf16"]
        tf = fl / (ms * 1e-3) / 1e12
        res[name] = {"workload": f"featmap {B}x{H}x{n} d={d} m={m} p={p} t={t} bf16 phi",
                     "kernel_ms": {k: round(v, 4) for k, v in kern.items()},
                     "tflop_per_launch": round(fl / 1e12, 4), "achieved_tflops": round(tf, 1),
                     "peak_tflops": PEAK_BF16_TFLOPS, "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        del th, ws, out
    return res


def featmap_backward(steps, torch, lib, t=4):
    """The feature map's backward (dX and dTheta from a bf16 dphi) at the long
    workload's geometry: 1 x 32 heads x 65536 rows, d = 128, m = 256, p = 2,
    t = 4 (or t = 1, the BASED-shaped map), squared, per-head Theta.
    Algorithmic work is three products of 2 d m p t flops per row (Y = X Theta,
    dY Theta^T, X^T dY); each of the two kernels recomputes Y once instead of
    reading it back."""
    g = torch.Generator(device="cpu").manual_seed(7)
    B, H, n, d, m, p = 1, 32, 65536, 128, 256, 2
    X = (torch.randn(B, H, n, d, generator=g) / d ** 0.5).to(torch.bfloat16).to("cuda")
    th = (torch.randn(H, p, t, d, m, generator=g) / d ** 0.5).to(torch.bfloat16).to("cuda")
    G = torch.randn(B, H, n, m, generator=g).to(torch.bfloat16).to("cuda")
    shape = lib.make_shape(batch=B, heads=H, n=n, d=d, dv=1, m=m, p=p, t=t, square=True,
                           in_dtype=lib.BF16, out_dtype=lib.BF16)
    ws = torch.empty(max(1, lib.llops_workspace_bytes(shape, lib.ENTRY_FEATMAP_BWD)),
                     dtype=torch.uint8, device="cuda")
    dX = torch.empty((B, H, n, d), dtype=torch.float32, device="cuda")
    dth = torch.empty(th.shape, dtype=torch.float32, device="cuda")

    def call():
        lib.llops_featmap_bwd(X, th, G, square=True, dX=dX, dtheta=dth, workspace=ws)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    timer = lib.KernelTimer(capacity=4 * steps)
    with timer:
        for _ in range(steps):
            call()
    torch.cuda.synchronize()
    kern = {k: sum(v) / len(v) for k, v in timer.durations_ms().items()}
    unit = 2.0 * B * H * n * d * m * p * t
    fl = 3 * unit
    tf = fl / (ms * 1e-3) / 1e12
    res = {"workload": f"featmap backward {B}x{H}x{n} d={d} m={m} p={p} t={t} squared, "
                       "bf16 X/Theta/dphi, fp32 dX/dTheta",
           "ms_per_call": round(ms, 4), "tokens_per_s": round(B * n / (ms * 1e-3), 1),
           "algorithmic_tflop": round(fl / 1e12, 4), "achieved_tflops": round(tf, 1),
           "peak_tflops": PEAK_BF16_TFLOPS, "frac": round(tf / PEAK_BF16_TFLOPS, 4),
           "kernel_ms": {k: round(v, 4) for k, v in kern.items()}}
    # per kernel: dX does Y and dY Theta^T; dTheta does Y and X^T dY
    for k, mult in (("featmap_bwd_dx", 2), ("featmap_bwd_dth", 2)):
        if k in kern:
            a = mult * unit / (kern[k] * 1e-3) / 1e12
            res[k] = {"algorithmic_tflop": round(mult * unit / 1e12, 4),
                      "achieved_tflops": round(a, 1), "frac": round(a / PEAK_BF16_TFLOPS, 4)}
    del X, th, G, ws, dX, dth
    return res


def causal_backward(steps, torch, lib):
    """The causal attention's full backward (llops_linattn_causal_bwd: feature
    maps, the attention chain rule as causal passes, the feature-map backward
    of both sides) at the long workload's geometry: 1 x 32 x 65536, d = dv =
    128, m = 256, p = 2, t = 4, squared, normalised. Synthetic bf16 inputs and
    an fp32 N(0,1) upstream gradient."""
    g = torch.Generator(device="cpu").manual_seed(11)
    B, H, n, d, dv, m, p, t = 1, 32, 65536, 128, 128, 256, 2, 4
    mk = lambda *shape, scale=1.0: (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16).to("cuda")
    Q, K = mk(B, H, n, d, scale=d ** -0.5), mk(B, H, n, d, scale=d ** -0.5)
    V = mk(B, H, n, dv)
    tq, tk = mk(H, p, t, d, m, scale=d ** -0.5), mk(H, p, t, d, m, scale=d ** -0.5)
    dO = torch.randn(B, H, n, dv, generator=g).to("cuda")
    shape = lib.make_shape(batch=B, heads=H, n=n, d=d, dv=dv, m=m, p=p, t=t, square=True,
                           normalize=True, delta=1e-6)
    ws = torch.empty(lib.llops_workspace_bytes(shape, lib.ENTRY_CAUSAL_BWD), dtype=torch.uint8,
                     device="cuda")

    def call():
        return lib.llops_linattn_causal_bwd(Q, K, V, tq, tk, dO, square=True, normalize=True,
                                            delta=1e-6, workspace=ws)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    timer = lib.KernelTimer(capacity=64 * steps)
    with timer:
        for _ in range(steps):
            call()
    torch.cuda.synchronize()
    kern = {k: sum(v) / steps for k, v in timer.durations_ms().items()}  # ms per call
    res = {"workload": f"causal attention backward {B}x{H}x{n} d={d} dv={dv} m={m} p={p} t={t} "
                       "squared, normalised; bf16 in, fp32 dO and gradients",
           "ms_per_call": round(ms, 3), "tokens_per_s": round(B * n / (ms * 1e-3), 1),
           "workspace_GiB": round(ws.numel() / 2 ** 30, 2),
           "kernel_ms_per_call": {k: round(v, 3) for k, v in sorted(kern.items(), key=lambda kv: -kv[1])}}
    del Q, K, V, tq, tk, dO, ws
    return res


def linattn_backward(steps, torch, lib):
    """The non-causal attention's full backward (llops_linattn_bwd: feature
    maps, the attention chain rule as non-causal passes, the feature-map
    backward of both sides) at the long workload's geometry: 1 x 32 x 65536, d = dv =
    128, m = 256, p = 2, t = 4, squared, normalised. Synthetic bf16 inputs and
    an fp32 N(0,1) upstream gradient."""
    g = torch.Generator(device="cpu").manual_seed(13)
    B, H, n, d, dv, m, p, t = 1, 32, 65536, 128, 128, 256, 2, 4
    mk = lambda *shape, scale=1.0: (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16).to("cuda")
    Q, K = mk(B, H, n, d, scale=d ** -0.5), mk(B, H, n, d, scale=d ** -0.5)
    V = mk(B, H, n, dv)
    tq, tk = mk(H, p, t, d, m, scale=d ** -0.5), mk(H, p, t, d, m, scale=d ** -0.5)
    dO = torch.randn(B, H, n, dv, generator=g).to("cuda")
    shape = lib.make_shape(batch=B, heads=H, n=n, d=d, dv=dv, m=m, p=p, t=t, square=True,
                           normalize=True, delta=1e-6)
    ws = torch.empty(lib.llops_workspace_bytes(shape, lib.ENTRY_LINATTN_BWD), dtype=torch.uint8,
                     device="cuda")

    def call():
        return lib.llops_linattn_bwd(Q, K, V, tq, tk, dO, square=True, normalize=True,
                                     delta=1e-6, workspace=ws)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    timer = lib.KernelTimer(capacity=64 * steps)
    with timer:
        for _ in range(steps):
            call()
    torch.cuda.synchronize()
    kern = {k: sum(v) / steps for k, v in timer.durations_ms().items()}  # ms per call
    res = {"workload": f"non-causal attention backward {B}x{H}x{n} d={d} dv={dv} m={m} p={p} t={t} "
                       "squared, normalised; bf16 in, fp32 dO and gradients",
           "ms_per_call": round(ms, 3), "tokens_per_s": round(B * n / (ms * 1e-3), 1),
           "workspace_GiB": round(ws.numel() / 2 ** 30, 2),
           "kernel_ms_per_call": {k: round(v, 3) for k, v in sorted(kern.items(), key=lambda kv: -kv[1])}}
    del Q, K, V, tq, tk, dO, ws
    return res


def state_backward(steps, torch, lib):
    """Both causal backwards continued from an initial state
    (llops_linattn_causal_bwd_state, llops_linattn_gated_causal_bwd_state,
    which also return dS0 and dz0) at the long workload's geometry: 1 x 32 x
    65536, d = dv = 128, m = 256, p = 2, t = 4, squared, normalised; S0 ~
    0.01 N(0,1), z0 = |0.01 N(0,1)|; gated: log gates log(sigmoid(N(4, 1)))."""
    g = torch.Generator(device="cpu").manual_seed(14)
    B, H, n, d, dv, m, p, t = 1, 32, 65536, 128, 128, 256, 2, 4
    mk = lambda *shape, scale=1.0: (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16).to("cuda")
    Q, K = mk(B, H, n, d, scale=d ** -0.5), mk(B, H, n, d, scale=d ** -0.5)
    V = mk(B, H, n, dv)
    tq, tk = mk(H, p, t, d, m, scale=d ** -0.5), mk(H, p, t, d, m, scale=d ** -0.5)
    dO = torch.randn(B, H, n, dv, generator=g).to("cuda")
    S0 = (0.01 * torch.randn(B, H, m, dv, generator=g)).to("cuda")
    z0 = (0.01 * torch.randn(B, H, m, generator=g)).abs().to("cuda")
    lg = torch.nn.functional.logsigmoid(torch.randn(B, H, n, generator=g) + 4.0).to("cuda")
    shape = lib.make_shape(batch=B, heads=H, n=n, d=d, dv=dv, m=m, p=p, t=t, square=True,
                           normalize=True, delta=1e-6)
    ws = torch.empty(lib.llops_workspace_bytes(shape, lib.ENTRY_GATED_CAUSAL_BWD), dtype=torch.uint8,
                     device="cuda")
    calls = {
        "causal": lambda: lib.llops_linattn_causal_bwd_state(
            Q, K, V, tq, tk, dO, S0=S0, z0=z0, square=True, normalize=True, delta=1e-6,
            workspace=ws),
        "gated": lambda: lib.llops_linattn_gated_causal_bwd_state(
            Q, K, V, tq, tk, lg, dO, S0=S0, z0=z0, square=True, normalize=True, delta=1e-6,
            workspace=ws),
    }
    res = {"workload": f"causal and gated causal attention backward from an initial state {B}x{H}x{n} "
                       f"d={d} dv={dv} m={m} p={p} t={t} squared, normalised; bf16 in, fp32 dO, "
                       "S0, z0 and gradients (incl. dS0, dz0)"}
    for name, call in calls.items():
        for _ in range(2):
            call()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        res[name] = {"ms_per_call": round(ms, 3), "tokens_per_s": round(B * n / (ms * 1e-3), 1)}
    del Q, K, V, tq, tk, dO, S0, z0, lg, ws
    return res


def gated_backward(steps, torch, lib):
    """The gated causal attention's full backward (llops_linattn_gated_causal_bwd,
    with the log-gate gradient) at the long workload's geometry: 1 x 32 x 65536,
    d = dv = 128, m = 256, p = 2, t = 4, squared, normalised; log gates
    log(sigmoid(N(4, 1))). Synthetic bf16 inputs, fp32 N(0,1) upstream gradient."""
    g = torch.Generator(device="cpu").manual_seed(12)
    B, H, n, d, dv, m, p, t = 1, 32, 65536, 128, 128, 256, 2, 4
    mk = lambda *shape, scale=1.0: (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16).to("cuda")
    Q, K = mk(B, H, n, d, scale=d ** -0.5), mk(B, H, n, d, scale=d ** -0.5)
    V = mk(B, H, n, dv)
    tq, tk = mk(H, p, t, d, m, scale=d ** -0.5), mk(H, p, t, d, m, scale=d ** -0.5)
    dO = torch.randn(B, H, n, dv, generator=g).to("cuda")
    lg = torch.nn.functional.logsigmoid(torch.randn(B, H, n, generator=g) + 4.0).to("cuda")
    shape = lib.make_shape(batch=B, heads=H, n=n, d=d, dv=dv, m=m, p=p, t=t, square=True,
                           normalize=True, delta=1e-6)
    ws = torch.empty(lib.llops_workspace_bytes(shape, lib.ENTRY_GATED_CAUSAL_BWD),
                     dtype=torch.uint8, device="cuda")

    def call():
        return lib.llops_linattn_gated_causal_bwd(Q, K, V, tq, tk, lg, dO, square=True,
                                                  normalize=True, delta=1e-6, workspace=ws)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    timer = lib.KernelTimer(capacity=128 * steps)
    with timer:
        for _ in range(steps):
            call()
    torch.cuda.synchronize()
    kern = {k: sum(v) / steps for k, v in timer.durations_ms().items()}  # ms per call
    res = {"workload": f"gated causal attention backward {B}x{H}x{n} d={d} dv={dv} m={m} p={p} "
                       f"t={t} squared, normalised, log gates log(sigmoid(N(4,1))); bf16 in, fp32 "
                       "dO and gradients (incl. dlog_gate)",
           "ms_per_call": round(ms, 3), "tokens_per_s": round(B * n / (ms * 1e-3), 1),
           "workspace_GiB": round(ws.numel() / 2 ** 30, 2),
           "kernel_ms_per_call": {k: round(v, 3) for k, v in sorted(kern.items(), key=lambda kv: -kv[1])}}
    del Q, K, V, tq, tk, dO, lg, ws
    return res


def config_lines(steps, torch, lib):
    """Per-workload throughput next to the bf16 MFMA (or fp32) peak."""
    from learnable_polynomial_feature_amd.workloads import WORKLOADS
    res = {}
    for name in ("tiny_noncausal_f32", "causal_p2_m64", "causal_p3_m128"):
        w = WORKLOADS[name]
        log(f"config {name}")
        ms, kern, gms = bench_config(w, steps, 3, torch, lib)
        fl = attention_flops(w)
        tf = fl / (ms * 1e-3) / 1e12
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
        res[name] = {"ms_per_call": round(ms, 4), "us_per_call": round(ms * 1e3, 2),
                     "tokens_per_s": round(w.batch * w.n / (ms * 1e-3), 1),
                     "algorithmic_tflop": round(fl / 1e12, 5), "achieved_tflops": round(tf, 3),
                     "peak_tflops": peak, "frac": round(tf / peak, 5),
                     "kernel_ms": {k: round(v, 4) for k, v in kern.items()},
                     "kernel_sum_us": round(sum(kern.values()) * 1e3, 2),
                     "graph": {"us_per_call": round(gms * 1e3, 2),
                               "tokens_per_s": round(w.batch * w.n / (gms * 1e-3), 1),
                               "frac": round(fl / (gms * 1e-3) / 1e12 / peak, 5),
                               "note": "one call captured as a HIP graph and replayed"}}
    return res


def bench_decode(w, steps, torch, lib):
    """Prefix state from the GPU causal pass (untimed), then `steps` decode steps."""
    from learnable_polynomial_feature_amd.workloads import decode_prefix, decode_tokens, generate
    B, H, m, dv = w.batch, w.heads, w.m, w.dv
    th = generate(w.replace(n=1, batch=1))
    gq, gk = to_dev(th["theta_q"], torch, torch.bfloat16), to_dev(th["theta_k"], torch,
                                                                   torch.bfloat16)
    S = torch.empty((B, H, m, dv), dtype=torch.float32, device="cuda")
    z = torch.empty((B, H, m), dtype=torch.float32, device="cuda")
    kw = dict(square=w.square, normalize=w.normalize, delta=w.delta)
    rows = 16
    log(f"decode: building the {w.prefix}-token prefix state")
    for b0 in range(0, B, rows):
        pre = decode_prefix(w, batches=list(range(b0, min(B, b0 + rows))))
        Kp = to_dev(pre["K_pre"], torch, torch.bfloat16)
        Vp = to_dev(pre["V_pre"], torch, torch.bfloat16)
        del pre
        lib.llops_linattn_causal_fwd(Kp, Kp, Vp, gq, gk, chunk=w.chunk, S_final=S[b0:b0 + rows],
                                     z_final=z[b0:b0 + rows], **kw)
        torch.cuda.synchronize()
        del Kp, Vp
    log(f"decode: generating {steps} steps of tokens")
    tok = decode_tokens(w, steps)
    q = to_dev(tok["q"], torch, torch.bfloat16)
    k = to_dev(tok["k"], torch, torch.bfloat16)
    v = to_dev(tok["v"], torch, torch.bfloat16)
    # the tokens of a few slices spread over the batch rows and heads, for
    # the oracle's CPU baseline
    sample = [(b, h, tok["q"][:, b, h].copy(), tok["k"][:, b, h].copy(), tok["v"][:, b, h].copy())
              for b, h in ((0, 0), (45, 2), (90, 11), (127, 15), (18, 5), (63, 17), (108, 1),
                           (36, 13), (81, 26), (9, 31), (117, 30), (54, 29))
              if b < B and h < H]
    del tok
    out = torch.empty((B, H, dv), dtype=torch.float32, device="cuda")
    shape = lib.make_shape(batch=B, heads=H, n=1, d=w.d, dv=dv, m=m, p=w.p, t=w.t,
                           square=w.square, normalize=w.normalize, delta=w.delta)
    ws = torch.empty(lib.llops_workspace_bytes(shape, lib.ENTRY_DECODE), dtype=torch.uint8,
                     device="cuda")
    S_init, z_init = S.clone(), z.clone()
    for s in range(3):  # warmup, then restore the prefix state
        lib.llops_decode_step(q[s], k[s], v[s], gq, gk, S, z, out=out, workspace=ws, **kw)
    S.copy_(S_init)
    z.copy_(z_init)
    torch.cuda.synchronize()
    # the whole loop captured once as a HIP graph (no host launch work per
    # step), replayed from the prefix state
    log(f"decode: capturing {steps} steps as one graph")
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        for s in range(steps):
            lib.llops_decode_step(q[s], k[s], v[s], gq, gk, S, z, out=out, workspace=ws, **kw)
    torch.cuda.synchronize()
    S.copy_(S_init)
    z.copy_(z_init)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    graph.replay()
    t1.record()
    torch.cuda.synchronize()
    graph_ms = t0.elapsed_time(t1) / steps
    del graph
    S.copy_(S_init)
    z.copy_(z_init)
    del S_init, z_init
    torch.cuda.synchronize()
    log(f"decode: timing {steps} steps")
    # a step is a few short kernels: the per-launch events of the kernel timer
    # would sit between them, so the steps are timed without it and the
    # kernels in a second pass over the same tokens
    t0.record()
    for s in range(steps):
        lib.llops_decode_step(q[s], k[s], v[s], gq, gk, S, z, out=out, workspace=ws, **kw)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    kstep = min(steps, 200)
    timer = lib.KernelTimer(capacity=8 * kstep)
    with timer:
        for s in range(kstep):
            lib.llops_decode_step(q[s], k[s], v[s], gq, gk, S, z, out=out, workspace=ws, **kw)
    torch.cuda.synchronize()
    kern = {kk: sum(vv) / len(vv) for kk, vv in timer.durations_ms().items()}
    # the gated step over the same tokens, with per-step log gates
    from learnable_polynomial_feature_amd.workloads import decode_step_gates
    gsteps = min(steps, 200)
    lg = torch.from_numpy(np.stack([decode_step_gates(w, s) for s in range(gsteps)])).to("cuda")
    for s in range(3):
        lib.llops_gated_decode_step(q[s], k[s], v[s], gq, gk, lg[s], S, z, out=out, workspace=ws,
                                    **kw)
    torch.cuda.synchronize()
    t0.record()
    for s in range(gsteps):
        lib.llops_gated_decode_step(q[s], k[s], v[s], gq, gk, lg[s], S, z, out=out, workspace=ws,
                                    **kw)
    t1.record()
    torch.cuda.synchronize()
    gms = t0.elapsed_time(t1) / gsteps
    timer = lib.KernelTimer(capacity=8 * gsteps)
    with timer:
        for s in range(gsteps):
            lib.llops_gated_decode_step(q[s], k[s], v[s], gq, gk, lg[s], S, z, out=out,
                                        workspace=ws, **kw)
    torch.cuda.synchronize()
    gkern = {kk: sum(vv) / len(vv) for kk, vv in timer.durations_ms().items()}
    gated = {"graph_ms_per_step": graph_ms, "steps": gsteps, "ms_per_step": round(gms, 4),
             "tokens_per_s": round(B / (gms * 1e-3), 1),
             "GBps": round(decode_bytes(w) / (gms * 1e-3) / 1e9, 1),
             "kernel_ms": {kk: round(vv, 4) for kk, vv in gkern.items()}}
    return ms, kern, gated, sample


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline(w, budget_s, min_s=0.5):
    """The fp64 oracle, as it stands, on whole (batch, head) sequences of the
    workload: causal_chunked at the workload's chunk, or linattn for the
    non-causal one. Slices run in order until about budget_s of oracle time
    (at least one; all of them, repeated to at least min_s, when they fit),
    and the full call's time is extrapolated from the slices done. Input
    generation is not timed."""
    from oracle import llops_oracle as O
    from learnable_polynomial_feature_amd.workloads import generate
    slices = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    kw = dict(square=w.square, normalize=w.normalize, delta=w.delta)
    done, elapsed = 0, 0.0
    cache = {}
    while (done < len(slices) and (elapsed < budget_s or done == 0)) or \
            (done % len(slices) == 0 and elapsed < min_s):
        b, h = slices[done % len(slices)]
        if (b, h) not in cache:
            x = generate(w, heads=[h], batches=[b])
            args = (x["Q"][0, 0], x["K"][0, 0], x["V"][0, 0], x["theta_q"][0], x["theta_k"][0])
            if len(slices) <= 64:  # small workloads: keep the inputs for repeated passes
                cache[(b, h)] = args
        else:
            args = cache[(b, h)]
        t = time.perf_counter()
        if w.causal:
            O.causal_chunked(*args, chunk=w.chunk, **kw)
        else:
            O.linattn(*args, **kw)
        elapsed += time.perf_counter() - t
        done += 1
    full_call = elapsed / done * len(slices)
    if done >= len(slices):
        what = (f"all {len(slices)} (batch, head) sequences, {done // len(slices)} pass(es), "
                f"{elapsed:.2f} s")
    else:
        what = (f"{done} of {len(slices)} (batch, head) sequences at full length ({w.n} tokens "
                f"each), {elapsed:.1f} s; full call extrapolated x{len(slices)}/{done}")
    return {"value": round(w.batch * w.n / full_call, 1), "unit": "tokens/s",
            "cores": int(_blas_threads()), "kind": "oracle",
            "sample": f"{w.name}: {what}; fp64 numpy oracle"}


def cpu_baseline_decode(w, sample, budget_s):
    """The fp64 oracle's decode (every step of the run, token by token) on
    (batch, head) slices of the decode workload, from the oracle's own
    prefix state (built untimed), until about budget_s; the full step's time
    is extrapolated to all batch x heads slices. sample: [(b, h, q, k, v)]
    with the slice's per-step tokens [steps, d|dv] as the GPU ran them."""
    from oracle import llops_oracle as O
    from learnable_polynomial_feature_amd.workloads import decode_prefix, theta_head
    kw = dict(square=w.square, normalize=w.normalize, delta=w.delta)
    done, elapsed, steps = 0, 0.0, 0
    for b, h, q, k, v in sample:
        if done and elapsed >= budget_s:
            break
        pre = decode_prefix(w, heads=[h], batches=[b])
        tq, tk = theta_head(w, "q", h), theta_head(w, "k", h)
        S0, z0 = O.state_from_prefix(pre["K_pre"][0, 0], pre["V_pre"][0, 0], tk,
                                     square=w.square)
        t = time.perf_counter()
        O.decode(S0, z0, q, k, v, tq, tk, **kw)
        elapsed += time.perf_counter() - t
        done += 1
        steps = len(q)
    per_step = elapsed / done / steps * w.batch * w.heads  # one step of every slice
    return {"value": round(w.batch / per_step, 1), "unit": "tokens/s",
            "cores": int(_blas_threads()), "kind": "oracle",
            "sample": f"{w.name}: {done} of {w.batch * w.heads} (batch, head) slices x {steps} "
                      f"steps, {elapsed:.1f} s; full step extrapolated "
                      f"x{w.batch * w.heads}/{done}; fp64 numpy oracle"}


def _power_node(torch):
    """The amdgpu hwmon power reading (microwatts) of cuda:0's PCI device, or
    None when sysfs does not expose it."""
    import glob
    props = torch.cuda.get_device_properties(0)
    bus = getattr(props, "pci_bus_id", None)
    dev = getattr(props, "pci_device_id", None)
    dom = getattr(props, "pci_domain_id", 0) or 0
    cands = []
    if bus is not None and dev is not None:
        base = f"/sys/bus/pci/devices/{dom:04x}:{bus:02x}:{dev:02x}.0/hwmon/hwmon*/"
        cands += sorted(glob.glob(base + "power1_average")) + sorted(glob.glob(base + "power1_input"))
    if not cands:  # a single amdgpu card in sysfs is this one
        nodes = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_average")) or \
            sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input"))
        if len(nodes) == 1:
            cands = nodes
    for f in cands:
        try:
            int(open(f).read())
            return f
        except (OSError, ValueError):
            continue
    return None


def power_account(node, fn, steps_per_call, secs, torch):
    """Average board power (W) while fn() runs back to back for about secs,
    sampled every 5 ms from another thread; joules per step = W x s/step."""
    import threading
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                samples.append(int(open(node).read()) * 1e-6)
            except (OSError, ValueError):
                pass
            time.sleep(0.005)
    fn()
    torch.cuda.synchronize()
    th = threading.Thread(target=sample, daemon=True)
    t0 = time.perf_counter()
    th.start()
    calls = 0
    while time.perf_counter() - t0 < secs:
        fn()
        calls += 1
        if calls % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stop.set()
    th.join()
    steps = calls * steps_per_call
    watts = sum(samples[len(samples) // 5:]) / max(1, len(samples) - len(samples) // 5)
    return {"watts": round(watts, 1), "ms_per_step": round(wall / steps * 1e3, 4),
            "joules_per_step": round(watts * wall / steps, 4), "samples": len(samples)}


def mfma_calibration(torch, size=8192, reps=10):
    """What a plain dense bf16 matrix product (torch.matmul, hipBLASLt)
    reaches on this board under its power cap: context for the MFMA rooflines
    (the nominal 2.5 PFLOP/s assumes 2.4 GHz)."""
    a = torch.randn(size, size, device="cuda").to(torch.bfloat16)
    b = torch.randn(size, size, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        a @ b
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        a @ b
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    tf = 2.0 * size ** 3 / (ms * 1e-3) / 1e12
    del a, b
    return {"op": f"torch.matmul bf16 {size}x{size}x{size}", "ms": round(ms, 4),
            "achieved": round(tf, 1), "unit": "TFLOP/s", "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def copy_probe(torch, nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size: under rocprofv3 --pmc its
    FETCH_SIZE / WRITE_SIZE read what `nbytes` of HBM traffic reads as."""
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"copy probe: {reps} x {nbytes} bytes")
    del x, y


def load_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None if absent or taken on a different kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[kernel]
    except (OSError, KeyError, ValueError):
        return None
    src = os.path.join(ROOT, "learnable_polynomial_feature_amd", "csrc", rec["source"])
    try:
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    if sha != rec["source_sha256"]:
        return None
    return rec["hbm_bytes_per_launch"]


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    from learnable_polynomial_feature_amd import _lib as lib
    from learnable_polynomial_feature_amd.workloads import WORKLOADS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    lib.library()
    if args.copy_probe:
        copy_probe(torch)
    w = WORKLOADS[args.workload]
    if w.steps:
        raise SystemExit("use the default causal workload; decode is reported in the same line")

    ms, kern, (cargs, cws) = bench_causal(w, args.steps, args.warmup, torch, lib)
    tokens = w.batch * w.n
    flops = causal_flops(w)
    # the dominant kernel (longest average launch) against the bf16 MFMA
    # peak, its duration from the HIP events recorded around each launch on
    # the launch stream; every kernel of the step beside it
    kfl = step_kernel_flops(w, kern)
    per_kernel = {k: {"avg_ms": round(kern[k], 4), "tflop_per_launch": round(f / 1e12, 4),
                      "frac": round(f / (kern[k] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
                  for k, f in kfl.items()}
    roofline = None
    if kfl:
        dom = max(kfl, key=lambda k: kern[k])
        ach = kfl[dom] / (kern[dom] * 1e-3) / 1e12
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": load_traffic(dom),
                    "avg_ms": round(kern[dom], 4), "flops_per_launch": kfl[dom]}
    line = {
        "metric": "causal LLoPS fwd tokens/sec at n=65536,p=2,t=4,m=256; % MFMA peak; decode GB/s",
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "n": w.n, "d": w.d,
                   "dv": w.dv, "p": w.p, "t": w.t, "m": w.m, "chunk": w.chunk,
                   "square": w.square, "normalize": w.normalize, "delta": w.delta,
                   "parallelism": "single-gpu"},
        "mfma_frac_step": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "algorithmic_tflop_per_step": round(flops / 1e12, 4),
        # the whole step (every kernel of one call) against the same peak; the
        # intra-chunk triangle is counted at the 32-token chunk the kernels run
        "step_roofline": {"bound": "mfma", "achieved": round(flops / (ms * 1e-3) / 1e12, 2),
                          "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "flops_per_step": flops, "intra_chunk_tokens": kernel_chunk(w)},
        "kernel_ms": {k: round(v, 4) for k, v in kern.items()},
        "kernel_mfma": per_kernel,
        "roofline": roofline,
    }
    if not args.no_decode:
        wd = WORKLOADS["decode_b128_h32"]
        dms, dkern, dgated, dsample = bench_decode(wd, args.decode_steps, torch, lib)
        graph_ms = dgated.pop("graph_ms_per_step")
        gb = decode_bytes(wd) / (dms * 1e-3) / 1e9
        st_ms = dkern.get("decode_state")
        st_gb = decode_state_bytes(wd) / (st_ms * 1e-3) / 1e9 if st_ms else None
        line["decode"] = {
            "workload": wd.name, "steps": args.decode_steps, "ms_per_step": round(dms, 4),
            "tokens_per_s": round(wd.batch / (dms * 1e-3), 1),
            "GBps": round(gb, 1), "hbm_frac": round(gb / PEAK_HBM_GBPS, 4),
            "graph": {"ms_per_step": round(graph_ms, 4),
                      "tokens_per_s": round(wd.batch / (graph_ms * 1e-3), 1),
                      "GBps": round(decode_bytes(wd) / (graph_ms * 1e-3) / 1e9, 1),
                      "hbm_frac": round(decode_bytes(wd) / (graph_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                      "note": "the whole loop captured once as a HIP graph and replayed"},
            "kernel_ms": {k: round(v, 4) for k, v in dkern.items()},
            "roofline": None if st_gb is None else {
                "kernel": "decode_state", "bound": "hbm", "achieved": round(st_gb, 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(st_gb / PEAK_HBM_GBPS, 4),
                "traffic": load_traffic("decode_state"),
                "bytes_per_launch": decode_state_bytes(wd)},
            "gated": dgated,
        }
    if args.power:
        node = _power_node(torch)
        if node is None:
            line["power"] = {"note": "no amdgpu hwmon power node for this device"}
        else:
            log(f"power: {node}")
            out_p = torch.empty((w.batch, w.heads, w.n, w.dv), dtype=torch.float32, device="cuda")
            kwp = dict(square=w.square, normalize=w.normalize, delta=w.delta, chunk=w.chunk,
                       out=out_p, workspace=cws)
            idle = []
            for _ in range(100):
                idle.append(int(open(node).read()) * 1e-6)
                time.sleep(0.005)
            acct = {"node": node, "idle_watts": round(sum(idle) / len(idle), 1)}
            try:
                acct["cap_watts"] = int(open(os.path.join(os.path.dirname(node),
                                                          "power1_cap")).read()) * 1e-6
            except (OSError, ValueError):
                pass
            prev = os.environ.get("LLOPS_FUSED_Q")
            for label, flag in (("two_kernel", "0"), ("fused", "1"), ("two_kernel_again", "0")):
                os.environ["LLOPS_FUSED_Q"] = flag
                acct[label] = power_account(
                    node, lambda: lib.llops_linattn_causal_fwd(*cargs, **kwp), 1, 8.0, torch)
            if prev is None:
                del os.environ["LLOPS_FUSED_Q"]
            else:
                os.environ["LLOPS_FUSED_Q"] = prev
            line["power"] = acct
            del out_p
    if "attn_out_fq" in kern:
        log("two-kernel causal path")
        line["two_kernel_path"] = bench_other_path(w, 10, torch, lib, cargs, cws, False)
    else:
        log("fused causal path")
        line["fused_path"] = bench_other_path(w, 10, torch, lib, cargs, cws, True)
    if not args.no_gated:
        log("gated causal")
        line["gated"] = bench_gated(w, 10, torch, lib, cargs, cws)
    del cargs, cws
    if not args.no_configs:
        line["configs"] = config_lines(20, torch, lib)
        log("feature-map variants")
        line["variants"] = featmap_variants(10, torch, lib)
        log("feature-map backward")
        line["featmap_backward"] = featmap_backward(10, torch, lib)
        line["featmap_backward_t1"] = featmap_backward(10, torch, lib, t=1)
        log("causal attention backward")
        line["causal_backward"] = causal_backward(3, torch, lib)
        log("gated causal attention backward")
        line["gated_backward"] = gated_backward(3, torch, lib)
        log("non-causal attention backward")
        line["linattn_backward"] = linattn_backward(3, torch, lib)
        log("attention backward from an initial state")
        line["state_backward"] = state_backward(3, torch, lib)
    if not args.no_configs:
        log("dense bf16 matmul calibration")
        line["mfma_calibration"] = mfma_calibration(torch)
    if not args.no_cpu_baseline:
        # the oracle timed on this host beside every workload's GPU figure
        log("cpu baseline (fp64 oracle)")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds * 0.5)
        if "configs" in line:
            for name in line["configs"]:
                line["configs"][name]["cpu_baseline"] = cpu_baseline(WORKLOADS[name],
                                                                     args.cpu_seconds / 8)
        if "decode" in line:
            line["decode"]["cpu_baseline"] = cpu_baseline_decode(
                WORKLOADS["decode_b128_h32"], dsample, args.cpu_seconds / 3)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
