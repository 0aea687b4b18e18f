#!/usr/bin/env python3
"""Throughput of the selective state space hot path on one MI355X.

Default workload (the headline): the Mamba-2.8b-shaped selective scan,
batch 4 x d_inner 5120 x d_state 16 x L 8192, bf16 u/delta/B/C/z/y, fp32 A/D
and state.  One step = one mss_selective_scan_fwd call over the whole batch
(all of its kernels), inputs resident in HBM before the timed region.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

prints ONE JSON line: state updates/s (B*L*D*N per second), the roofline of
the dominant kernel (algorithmic bytes / event-timed launch duration against
8 TB/s HBM3E) and the fp64 CPU oracle's throughput on a bounded sample of the
same workload, timed on this host's cores.

Other workloads (measured for the record, not the headline):
  scan_130m    b8 x d1536 x N16 x L2048, fp32 I/O
  decode_2p8b  b256 x d5120 x N16 one-token steps, bf16 I/O; one step = 1000 tokens
  ssd_2p8b     b2 x L16384 x H80 x P64 x N128, chunk 256 (Mamba-2 SSD)
  scan_m2shape the Mamba-1 scan on ssd_2p8b's shape: b2 x d5120 (80 heads of
               64 channels) x N128 x L16384, A and delta shared within a head
  scan_2p8b_bwd  the backward (gradients of u, delta, A, B, C, D, z) of the
               headline scan, one mss_selective_scan_bwd call per step
  ssd_2p8b_bwd the backward of ssd_2p8b (gradients of x, delta, A, B, C), one
               mss_ssd_chunk_bwd call per step
  scan_2p8b_fused  the headline scan fed by its prologue (u from the silu of
               the causal 4-tap convolution of x, delta = softplus(raw + bias))
  decode_m3    Mamba-3 generation: b128 x 80 heads x P64 x N128, MIMO rank 4,
               complex (rotating) fp32 state, trapezoid input, bf16 I/O; one
               step = 100 consecutive tokens
  copy         a plain 1 GiB device copy (calibrates the HBM byte counters)

--seqlen L and --batch B (scan and SSD workloads) time the same workload at
another sequence length or batch: the preset's inputs are drawn as usual and
repeated (or cut) along L or the batch on the device.  Such lines carry no
traffic figure (the counters were taken at the preset shape) and no CPU
baseline.  --dstate N (scan_2p8b, scan_130m, scan_2p8b_bwd, scan_2p8b_fused)
draws the preset's inputs at d_state N instead; such lines carry no traffic
figure either, but keep the CPU baseline (the oracle at the same shape).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
# fp32 vector arithmetic: 256 CUs x 4 SIMDs x 16 lanes x 2 flops (FMA) x 2.4 GHz
# = 78.6 TFLOP/s without packed fp32 (kept out of the library's code), 157.3
# with it; bf16 dense MFMA 2.5 PFLOP/s.
ALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
ALU_PEAK_PACKED_TFLOPS = 2 * ALU_PEAK_TFLOPS
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "state updates/s (B*L*D*N) + % HBM roofline, Mamba-2.8b-shaped scan"


SCAN_WORKLOADS = ("scan_2p8b", "scan_130m", "scan_2p8b_bwd", "scan_2p8b_fused", "scan_2p8b_fused_bwd")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="scan_2p8b",
                    choices=["scan_2p8b", "scan_130m", "decode_2p8b", "ssd_2p8b", "ssd_2p8b_bwd", "scan_m2shape",
                             "scan_2p8b_bwd", "scan_2p8b_fused", "scan_2p8b_fused_bwd", "decode_m3", "copy"])
    ap.add_argument("--seqlen", type=int, default=0,
                    help="scan/SSD workloads: sequence length (inputs repeated along L); 0 = the preset's")
    ap.add_argument("--batch", type=int, default=0,
                    help="scan/SSD workloads: batch (inputs repeated along the batch); 0 = the preset's")
    ap.add_argument("--dstate", type=int, default=0,
                    help="selective scan workloads (forward, fused, backward): d_state in place of the preset's, "
                         "inputs drawn for that shape; 0 = the preset's")
    ap.add_argument("--force-general-decay", action="store_true",
                    help="scan: per-state exp decay even where A has the S4D-real structure")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    return ap.parse_args()


# ----------------------------------------------------------- byte counts ----
def scan_bytes(b, d, n, L, es):
    """Algorithmic bytes: u, delta, z read and y written once ([b,d,L]), B and C
    read once ([b,n,L]), A [d,n] and D [d] fp32 read once."""
    return 4 * b * d * L * es + 2 * b * n * L * es + d * n * 4 + d * 4


def scan_flops(b, d, n, L):
    """Algorithmic fp32 flops of the forward: per state update the decay (one
    multiply, or one exp), B*x, the update h = a*h + Bx (an FMA, 2 flops) and
    the readout C*h accumulated (2 flops); per (b, d, l) x = delta*u (1), the
    skip D*u added (2), silu(z) (4: negate, exp, add, divide) and the gate (1)."""
    return b * d * L * (6 * n + 8)


def scan_fused_flops(b, d, n, L):
    """The forward's flops plus the prologue per (b, d, l): the 4-tap
    convolution with bias (9), its silu (4), delta_raw + bias (1) and softplus
    (5: max, abs, exp, log1p, add)."""
    return scan_flops(b, d, n, L) + b * d * L * 19


def ssd_mfma_flops(b, L, H, P, N, Q):
    """Dense-tile matrix flops of the chunked SSD with 64-step blocks: per block
    and head C S^T (64x64 over N), the decay-masked diagonal block as a full
    64x64 tile times x (64x64 over 64) and the state update B^T (w x) (N x P
    over 64), plus C B^T per block and group (64x64 over N)."""
    blocks = b * (-(-L // 64))
    per_head = 2 * 64 * P * N + 2 * 64 * 64 * P + 2 * N * P * 64
    return blocks * (H * per_head + 2 * 64 * 64 * N)


def scan_fused_bytes(b, d, n, L, es):
    """The scan's bytes with x and the raw delta in place of u and delta, plus
    the taps [d,4] and the two biases [d] (fp32) read once."""
    return scan_bytes(b, d, n, L, es) + d * 4 * 4 + 2 * d * 4


def scan_bwd_bytes(b, d, n, L, es):
    """Algorithmic bytes of the backward: u, delta, z, dy read and du, ddelta,
    dz written once ([b,d,L]); B, C read and dB, dC written once ([b,N,L]); A,
    D read and dA, dD written once (fp32)."""
    return 7 * b * d * L * es + 4 * b * n * L * es + 2 * (d * n * 4 + d * 4)


def decode_step_bytes(b, d, n, es):
    """Per token step: state read + written (fp32), u/delta/z/y, B/C, A, D."""
    return 2 * b * d * n * 4 + 4 * b * d * es + 2 * b * n * es + d * n * 4 + d * 4


def mamba3_step_bytes(cfg, es):
    """Per token step: the state read and written (fp32, re and im when
    complex); x, z, y and x_prev [b,H,R,P]; B, C and B_prev [b,G,R,N]; delta
    [b,H]; A, D [H] and theta [H,N] fp32."""
    b, H, P, G, N, R = cfg.batch, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, cfg.rank
    state = b * H * P * N * 4 * (2 if cfg.complex_state else 1)
    return (2 * state + (4 if cfg.trapezoid else 3) * b * H * R * P * es + (3 if cfg.trapezoid else 2) * b * G * R * N * es
            + b * H * 4 + 2 * H * 4 + (H * N * 4 if cfg.complex_state else 0))


def ssd_bwd_mfma_flops(b, L, H, P, N):
    """Dense-tile matrix flops of the SSD backward: the forward pass with
    64-step chunks (ssd_mfma_flops), then per 64-step block and head the
    block's adjoint part C^T (e dy) (N x P over 64), W = dy x^T (64x64 over
    P), (G B)^T = E B^T + dy^T (M o K) (P x 64 over N and over 64),
    (x^T G)^T = E^T x^T + C^T (M o W) (N x 64 over P and over 64) and
    (h^T dy)^T = S^T dy^T + B^T (M o W^T) (N x 64 over P and over 64), plus
    K = C B^T per block and group (64x64 over N)."""
    blocks = b * (-(-L // 64))
    per_head = 4 * (2 * N * P * 64) + 2 * (2 * 64 * 64 * P) + 2 * (2 * N * 64 * 64)
    return ssd_mfma_flops(b, L, H, P, N, 64) + blocks * (H * per_head + 2 * 64 * 64 * N)


def ssd_bwd_bytes(b, L, H, P, G, N, es):
    """Algorithmic bytes of the SSD backward: x, B, C read once (bf16), delta,
    dy read once (fp32), A read once; dx, ddelta, dB, dC, dA written once
    (fp32)."""
    return (b * L * H * P * (es + 4 + 4) + b * L * H * 8 + b * L * G * N * (2 * es + 2 * 4) + 2 * H * 4)


def ssd_bytes(b, L, H, P, G, N, es):
    """x and B, C read once (bf16), delta (fp32), A, y written once (fp32)."""
    return b * L * H * P * es + 2 * b * L * G * N * es + b * L * H * 4 + H * 4 + b * L * H * P * 4


# ------------------------------------------------------- traffic record -----
def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "selective_state_space_27_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload, files):
    """HBM bytes per launch from the committed counter summary, or None when the
    summary is missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != kernel_source_hash(files):
        return None
    return float(m_val.group(1))


# ------------------------------------------------------------ workloads -----
def to_dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(a).to("cuda:0")


STEP_TIMES = {}  # per-step event times of the last timed region (median, p10, p90)


def time_region(torch, fn, steps, warmup):
    """Event-timed region on the current stream (the library launches there):
    ms per step over the whole region; an event between consecutive steps
    also gives each step's own time (STEP_TIMES)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    STEP_TIMES.update({"ms_per_step_median": float(np.median(per)), "ms_per_step_p10": float(np.percentile(per, 10)),
                       "ms_per_step_p90": float(np.percentile(per, 90))})
    return ev[0].elapsed_time(ev[-1]) / steps  # ms per step


CPU_MIN_S = 10.0  # the oracle leg repeats its sample until at least this much wall time has passed


def repeat_timed(fn, min_s=CPU_MIN_S, max_reps=100000):
    """Calls fn until at least min_s seconds have passed; returns (calls, seconds)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_s or reps >= max_reps:
            return reps, dt


def host_cpus():
    """The host's CPUs as this process sees them: (threads the oracle uses,
    description).  Threads = the CPUs in this process's affinity mask, capped
    by a cgroup CPU quota when one is set (more threads than the quota would
    only time-slice)."""
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count() or 1
    quota = None
    try:
        q, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if q != "max":
            quota = max(1, -(-int(q) // int(period)))
    except (OSError, ValueError):
        pass
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    threads = min(nproc, quota) if quota else nproc
    return threads, {"nproc": nproc, "cgroup_cpu_quota": quota, "cpu_model": model}


def cpu_leg(all_fn, all_units, one_fn, one_units, unit, threads, info, sample_all, sample_one):
    """Times the oracle on all host threads (all_fn, at least CPU_MIN_S) and
    on one thread (one_fn on a smaller sample, at least CPU_MIN_S / 2)."""
    reps, dt = repeat_timed(all_fn)
    reps1, dt1 = repeat_timed(one_fn, CPU_MIN_S / 2)
    res = {"value": reps * all_units / dt, "unit": unit, "cores": threads, "kind": "oracle",
           "sample": f"{sample_all} {reps} times on {threads} threads; {dt:.2f} s wall, fp64 C oracle",
           "value_1thread": reps1 * one_units / dt1,
           "sample_1thread": f"{sample_one} {reps1} times on 1 thread; {dt1:.2f} s wall"}
    res.update(info)
    return res


def along_l(torch, t, L, dim):
    """Device tensor repeated (or cut) to length L along dimension `dim`."""
    reps = [1] * t.dim()
    reps[dim] = -(-L // t.shape[dim])
    return t.repeat(*reps).narrow(dim, 0, L).contiguous()


def bench_scan(args, torch, mss, I, cfg):
    x = I.scan_inputs(cfg)
    g = {k: to_dev(torch, x[k]) for k in ("u", "delta", "A", "B", "C", "D", "z")}
    io_dt = g["u"].dtype
    b, d, n, L = cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen
    if args.seqlen or args.batch:
        L, b = args.seqlen or L, args.batch or b
        for k in ("u", "delta", "B", "C", "z"):
            g[k] = along_l(torch, along_l(torch, g[k], L, 2), b, 0)
        torch.cuda.synchronize()
    ws = torch.empty(mss.selective_scan_workspace_size(b, d, n, L, io_dt), dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(g["u"])

    def step():
        mss.selective_scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], out=out, workspace=ws,
                               force_general_decay=args.force_general_decay)

    ms = time_region(torch, step, args.steps, args.warmup)
    updates = b * d * n * L
    es = 2 if cfg.io == "bf16" else 4
    nbytes = scan_bytes(b, d, n, L, es)
    res = {
        "metric": METRIC if cfg is I.SCAN_2P8B else "state updates/s (B*L*D*N), selective scan",
        "value": updates / (ms * 1e-3), "unit": "state updates/s", "ms_per_step": ms,
        "dtype": "f32",
        "config": {"workload": f"{cfg.name}: selective scan b={b} d_inner={d} d_state={n} L={L}, "
                               f"{cfg.io} u/delta/B/C/z/y, fp32 A/D/state",
                   "batch": b, "d_inner": d, "d_state": n, "seqlen": L, "io_dtype": cfg.io,
                   "decay": "per-state exp (forced)" if args.force_general_decay else
                            "one decay per (d, l) for all states (A equal over n, detected on device)"
                            if cfg.a_form == "head" else
                            "power chain (S4D-real structure detected on device)"},
    }
    if args.seqlen or args.batch:
        res["config"]["inputs"] = f"the preset's b={cfg.batch} L={cfg.seqlen} draw repeated or cut along b and L"
    res["alu_flops"] = scan_flops(b, d, n, L)
    files = ["scan.hip", "scan_layout.hpp", "common.hpp"]
    kernel = "scan_kernel (+ bc_transpose_kernel in the same timed call)"
    cpu = None
    if not args.no_cpu_baseline and not (args.seqlen or args.batch):
        import oracle
        f64 = lambda k: I.to_f64(x[k], cfg.io)  # the whole workload, repeated for at least CPU_MIN_S
        args64 = (f64("u"), f64("delta"), x["A"].astype(np.float64), f64("B"), f64("C"), x["D"].astype(np.float64),
                  f64("z"))
        th, info = host_cpus()
        d1 = max(1, d // 32)  # one thread: batch row 0, the first d/32 channels
        one = tuple(a[:1, :d1] if a.ndim == 3 and a.shape[1] == d else a[:1] if a.ndim == 3 else a[:d1]
                    for a in args64)
        cpu = cpu_leg(lambda: oracle.selective_scan(*args64, threads=th), b * d * n * L,
                      lambda: oracle.selective_scan(*one, threads=1), d1 * n * L, "state updates/s", th, info,
                      f"the whole workload (b={b}, d={d}, N={n}, L={L})", f"batch row 0, channels 0..{d1 - 1}")
    return res, nbytes, ms, kernel, files, cpu


def bench_scan_fused(args, torch, mss, I, cfg):
    x = I.scan_fused_inputs(cfg)
    keys = ("x", "conv_w", "conv_b", "delta_raw", "delta_bias", "A", "B", "C", "D", "z")
    g = {k: to_dev(torch, x[k]) for k in keys}
    io_dt = g["x"].dtype
    b, d, n, L = cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen
    ws = torch.empty(mss.selective_scan_workspace_size(b, d, n, L, io_dt), dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(g["x"])

    def step():
        mss.selective_scan_fwd_fused(*(g[k] for k in keys), conv_silu=True, softplus=True, out=out, workspace=ws)

    ms = time_region(torch, step, args.steps, args.warmup)
    es = 2 if cfg.io == "bf16" else 4
    res = {
        "metric": "state updates/s (B*L*D*N), selective scan fed by its prologue",
        "value": b * d * n * L / (ms * 1e-3), "unit": "state updates/s", "ms_per_step": ms, "dtype": "f32",
        "config": {"workload": f"{cfg.name}_fused: selective scan b={b} d_inner={d} d_state={n} L={L} whose u is "
                               "silu(causal 4-tap conv of x + bias) and delta softplus(delta_raw + bias), formed in "
                               f"the kernel; {cfg.io} x/delta_raw/B/C/z/y, fp32 taps/biases/A/D/state",
                   "batch": b, "d_inner": d, "d_state": n, "seqlen": L, "io_dtype": cfg.io},
    }
    res["alu_flops"] = scan_fused_flops(b, d, n, L)
    files = ["scan.hip", "scan_layout.hpp", "common.hpp"]
    kernel = "scan_kernel with the fused prologue (+ bc_transpose_kernel in the same timed call)"
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        f64 = lambda k: I.to_f64(x[k], cfg.io)
        th, info = host_cpus()
        xs, dr, Bs, Cs, zs = f64("x"), f64("delta_raw"), f64("B"), f64("C"), f64("z")
        d1 = max(1, d // 32)  # one thread: batch row 0, the first d/32 channels

        def call(bsl, dsl, t):
            return oracle.selective_scan_fused(xs[bsl, dsl], x["conv_w"][dsl], x["conv_b"][dsl], dr[bsl, dsl],
                                               x["delta_bias"][dsl], x["A"][dsl], Bs[bsl], Cs[bsl], x["D"][dsl],
                                               zs[bsl, dsl], conv_silu=True, softplus=True, threads=t)
        cpu = cpu_leg(lambda: call(slice(None), slice(None), th), b * d * n * L,
                      lambda: call(slice(0, 1), slice(0, d1), 1), d1 * n * L, "state updates/s", th, info,
                      f"the whole workload (b={b}, d={d}, N={n}, L={L}; prologue on one thread, scan on all)",
                      f"batch row 0, channels 0..{d1 - 1}")
    return res, scan_fused_bytes(b, d, n, L, es), ms, kernel, files, cpu


def bench_scan_bwd(args, torch, mss, I, cfg):
    x = I.scan_inputs(cfg)
    g = {k: to_dev(torch, x[k]) for k in ("u", "delta", "A", "B", "C", "D", "z")}
    dy_host = I.scan_grad_output(cfg)
    dy = to_dev(torch, dy_host)
    io_dt = g["u"].dtype
    b, d, n, L = cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen
    if args.seqlen or args.batch:
        L, b = args.seqlen or L, args.batch or b
        for k in ("u", "delta", "B", "C", "z"):
            g[k] = along_l(torch, along_l(torch, g[k], L, 2), b, 0)
        dy = along_l(torch, along_l(torch, dy, L, 2), b, 0)
        torch.cuda.synchronize()
    ws = torch.empty(mss.selective_scan_bwd_workspace_size(b, d, n, L, io_dt), dtype=torch.uint8, device="cuda:0")
    out = mss.selective_scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], dy=dy, workspace=ws)

    def step():
        mss.selective_scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], dy=dy, out=out,
                               workspace=ws)

    ms = time_region(torch, step, args.steps, args.warmup)
    es = 2 if cfg.io == "bf16" else 4
    res = {"metric": "state updates/s (B*L*D*N), selective scan backward", "value": b * d * n * L / (ms * 1e-3),
           "unit": "state updates/s", "ms_per_step": ms, "dtype": "f32",
           "config": {"workload": f"{cfg.name}_bwd: selective scan backward b={b} d_inner={d} d_state={n} L={L}, "
                                  f"{cfg.io} u/delta/B/C/z/dy and gradients, fp32 A/D/dA/dD/state",
                      "batch": b, "d_inner": d, "d_state": n, "seqlen": L, "io_dtype": cfg.io,
                      "gradients": "du, ddelta, dA, dB, dC, dD, dz"}}
    if args.seqlen or args.batch:
        res["config"]["inputs"] = f"the preset's b={cfg.batch} L={cfg.seqlen} draw repeated or cut along b and L"
    cpu = None
    if not args.no_cpu_baseline and not (args.seqlen or args.batch):
        import oracle
        f64 = lambda k: I.to_f64(x[k][:1], cfg.io)  # bounded sample: batch row 0, every channel, full L
        args64 = (f64("u"), f64("delta"), x["A"].astype(np.float64), f64("B"), f64("C"), x["D"].astype(np.float64),
                  f64("z"), None, I.to_f64(dy_host[:1], cfg.io))
        th, info = host_cpus()
        d1 = max(1, d // 64)
        one = tuple(None if a is None else a[:, :d1] if a.ndim == 3 and a.shape[1] == d else
                    a[:d1] if a.ndim in (1, 2) else a for a in args64)
        cpu = cpu_leg(lambda: oracle.selective_scan_bwd(*args64, threads=th), d * n * L,
                      lambda: oracle.selective_scan_bwd(*one, threads=1), d1 * n * L, "state updates/s", th, info,
                      f"batch row 0 of {b} (all {d} channels, full L={L}), backward",
                      f"batch row 0, channels 0..{d1 - 1}, backward")
    files = ["scan.hip", "scan_bwd.hip", "scan_layout.hpp", "common.hpp"]
    kernel = "scan_bwd_kernel (+ checkpoint forward and bwd_reduce_kernel in the same timed call)"
    return res, scan_bwd_bytes(b, d, n, L, es), ms, kernel, files, cpu


def bench_scan_fused_bwd(args, torch, mss, I, cfg):
    x = I.scan_fused_inputs(cfg)
    keys = ("x", "conv_w", "conv_b", "delta_raw", "delta_bias", "A", "B", "C", "D", "z")
    g = {k: to_dev(torch, x[k]) for k in keys}
    dy_host = I.scan_grad_output(cfg)
    dy = to_dev(torch, dy_host)
    io_dt = g["x"].dtype
    b, d, n, L = cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen
    flags = mss.MSS_FLAG_CONV_SILU | mss.MSS_FLAG_DELTA_SOFTPLUS
    ws = torch.empty(mss.lib().mss_selective_scan_fused_bwd_workspace_size(b, d, n, L, mss._io_code(io_dt), flags),
                     dtype=torch.uint8, device="cuda:0")

    def step():
        mss.selective_scan_fused_bwd(*(g[k] for k in keys), dy=dy, conv_silu=True, softplus=True, workspace=ws)

    ms = time_region(torch, step, args.steps, args.warmup)
    es = 2 if cfg.io == "bf16" else 4
    res = {"metric": "state updates/s (B*L*D*N), selective scan backward through its prologue",
           "value": b * d * n * L / (ms * 1e-3), "unit": "state updates/s", "ms_per_step": ms, "dtype": "f32",
           "config": {"workload": f"{cfg.name}_fused_bwd: backward of the scan fed by its prologue (silu "
                                  f"convolution, softplus delta) b={b} d_inner={d} d_state={n} L={L}, {cfg.io} "
                                  f"x/delta_raw/B/C/z/dy and gradients, fp32 taps, biases, A/D and their gradients",
                      "batch": b, "d_inner": d, "d_state": n, "seqlen": L, "io_dtype": cfg.io,
                      "gradients": "dx, ddelta_raw, dconv_w, dconv_b, ddelta_bias, dA, dB, dC, dD, dz"}}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        f64 = lambda k: I.to_f64(x[k][:1], cfg.io)  # bounded sample: batch row 0, every channel, full L
        args64 = (f64("x"), x["conv_w"], x["conv_b"], f64("delta_raw"), x["delta_bias"], x["A"].astype(np.float64),
                  f64("B"), f64("C"), x["D"].astype(np.float64), f64("z"), None)
        dy64 = I.to_f64(dy_host[:1], cfg.io)
        th, info = host_cpus()
        d1 = max(1, d // 64)
        one = tuple(None if a is None else a[:, :d1] if a.ndim == 3 and a.shape[1] == d else
                    a[:d1] if a.ndim in (1, 2) else a for a in args64)
        cpu = cpu_leg(lambda: oracle.selective_scan_fused_bwd(*args64, dy=dy64, conv_silu=True, softplus=True,
                                                              threads=th), d * n * L,
                      lambda: oracle.selective_scan_fused_bwd(*one, dy=dy64[:, :d1], conv_silu=True, softplus=True,
                                                              threads=1), d1 * n * L, "state updates/s", th, info,
                      f"batch row 0 of {b} (all {d} channels, full L={L}), fused backward",
                      f"batch row 0, channels 0..{d1 - 1}, fused backward")
    files = ["scan.hip", "scan_bwd.hip", "scan_fused_bwd.hip", "scan_layout.hpp", "common.hpp"]
    kernel = "scan_bwd_kernel (+ prologue, fp32 copies, checkpoint forward, reductions and the prologue's chain rule)"
    # The scan backward's bytes with x, delta_raw for u, delta and dx, ddelta_raw for du, ddelta, plus the taps.
    return res, scan_bwd_bytes(b, d, n, L, es) + 2 * d * 16 + 4 * d * 4, ms, kernel, files, cpu


def bench_decode(args, torch, mss, I):
    cfg = I.DECODE_2P8B
    st = I.decode_static(cfg)
    pool = [I.decode_step_inputs(cfg, s, st["dt"]) for s in range(I.DECODE_POOL)]
    dpool = [{k: to_dev(torch, p[k]) for k in ("u", "delta", "B", "C", "z")} for p in pool]
    h = to_dev(torch, I.decode_state0(cfg))
    A, D = to_dev(torch, st["A"]), to_dev(torch, st["D"])
    y = torch.empty((cfg.batch, cfg.dim), dtype=torch.bfloat16, device="cuda:0")

    def step():  # 1000 consecutive generation steps
        for s in range(cfg.steps):
            p = dpool[s % I.DECODE_POOL]
            mss.state_update(h, p["u"], p["delta"], A, p["B"], p["C"], D, p["z"], out=y)

    steps = max(1, args.steps // 10)
    ms = time_region(torch, step, steps, max(1, args.warmup // 5))
    b, d, n = cfg.batch, cfg.dim, cfg.dstate
    updates = b * d * n * cfg.steps
    res = {"metric": "state updates/s (B*D*N per token step), one-token generation", "value": updates / (ms * 1e-3),
           "unit": "state updates/s", "ms_per_step": ms, "dtype": "f32",
           "config": {"workload": f"{cfg.name}: state update b={b} d_inner={d} d_state={n}, 1000 consecutive tokens, "
                                  "bf16 u/delta/B/C/z/y, fp32 state in place", "batch": b, "d_inner": d, "d_state": n,
                      "tokens_per_step": cfg.steps}}
    nbytes = decode_step_bytes(b, d, n, 2)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        p64 = [{k: I.to_f64(p[k], "bf16") for k in ("u", "delta", "B", "C", "z")} for p in pool]
        state = {"h": I.decode_state0(cfg).astype(np.float64), "s": 0}
        th, info = host_cpus()
        b1 = max(1, b // 32)

        def token_step(nb, t):  # consecutive token steps, inputs cycling through the pool
            p = p64[state["s"] % I.DECODE_POOL]
            h, _ = oracle.state_update(state["h"][:nb], p["u"][:nb], p["delta"][:nb], st["A"], p["B"][:nb],
                                       p["C"][:nb], st["D"], p["z"][:nb], threads=t)
            state["h"][:nb] = h
            state["s"] += 1

        cpu = cpu_leg(lambda: token_step(b, th), b * d * n, lambda: token_step(b1, 1), b1 * d * n,
                      "state updates/s", th, info, f"all {b} batch rows, consecutive token steps",
                      f"batch rows 0..{b1 - 1}, consecutive token steps")
    # per-launch figures: one launch = one token step
    return res, nbytes, ms / cfg.steps, "state_update_kernel", ["state_update.hip", "common.hpp"], cpu


def bench_decode_m3(args, torch, mss, I):
    cfg = I.DECODE_M3
    st = I.mamba3_static(cfg)
    pool = [I.mamba3_step_inputs(cfg, s, st["dt"]) for s in range(I.DECODE_POOL)]
    dpool = [{k: to_dev(torch, p[k]) for k in ("x", "B", "C", "z", "delta")} for p in pool]
    h = to_dev(torch, st["h0"])
    A, D, th = to_dev(torch, st["A"]), to_dev(torch, st["D"]), to_dev(torch, st["theta"])
    y = torch.empty_like(dpool[0]["x"])

    def step():  # consecutive generation steps; x_prev, B_prev are the previous step's
        for s in range(cfg.steps):
            p, q = dpool[s % I.DECODE_POOL], dpool[(s - 1) % I.DECODE_POOL]
            mss.mamba3_state_update(h, p["x"], p["delta"], A, p["B"], p["C"], D, p["z"], x_prev=q["x"], B_prev=q["B"],
                                    theta=th, out=y)

    steps = max(1, args.steps // 10)
    ms = time_region(torch, step, steps, max(1, args.warmup // 5))
    b, H, P, N, R = cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, cfg.rank
    updates = b * H * P * N * cfg.steps
    res = {"metric": "state updates/s (B*H*P*N per token step), Mamba-3 generation", "value": updates / (ms * 1e-3),
           "unit": "state updates/s", "ms_per_step": ms, "dtype": "f32",
           "config": {"workload": f"{cfg.name}: Mamba-3 state update b={b} heads={H} headdim={P} d_state={N} "
                                  f"MIMO rank {R}, complex state, trapezoid input, {cfg.steps} consecutive tokens, "
                                  "bf16 x/B/C/z/y, fp32 state in place", "batch": b, "nheads": H, "headdim": P,
                      "d_state": N, "rank": R, "tokens_per_step": cfg.steps}}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        th_n, info = host_cpus()
        p64 = [{k: I.to_f64(p[k], "bf16") for k in ("x", "B", "C", "z")} | {"delta": p["delta"]} for p in pool]
        state = {"h": st["h0"].astype(np.float64), "s": 0}
        b1 = max(1, b // 32)

        def token_step(nb, t):
            p, q = p64[state["s"] % I.DECODE_POOL], p64[(state["s"] - 1) % I.DECODE_POOL]
            hn, _ = oracle.mamba3_step(state["h"][:nb], p["x"][:nb], p["delta"][:nb], st["A"], p["B"][:nb],
                                       p["C"][:nb], st["D"], p["z"][:nb], x_prev=q["x"][:nb], B_prev=q["B"][:nb],
                                       theta=st["theta"], complex_state=True, threads=t)
            state["h"][:nb] = hn
            state["s"] += 1

        cpu = cpu_leg(lambda: token_step(b, th_n), b * H * P * N, lambda: token_step(b1, 1), b1 * H * P * N,
                      "state updates/s", th_n, info, f"all {b} batch rows, consecutive token steps",
                      f"batch rows 0..{b1 - 1}, consecutive token steps")
    return res, mamba3_step_bytes(cfg, 2), ms / cfg.steps, "mamba3_step_kernel", ["mamba3.hip", "common.hpp"], cpu


def bench_ssd(args, torch, mss, I):
    cfg = I.SSD_2P8B
    x = I.ssd_inputs(cfg)
    g = {k: to_dev(torch, x[k]) for k in ("x", "delta", "A", "B", "C")}
    b, L, H, P, G, N, Q = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, cfg.chunk
    if args.seqlen or args.batch:
        L, b = args.seqlen or L, args.batch or b
        for k in ("x", "delta", "B", "C"):
            g[k] = along_l(torch, along_l(torch, g[k], L, 1), b, 0)
        torch.cuda.synchronize()
    ws = torch.empty(mss.ssd_workspace_size(b, L, H, P, G, N, Q), dtype=torch.uint8, device="cuda:0")
    out = torch.empty((b, L, H, P), dtype=torch.float32, device="cuda:0")

    def step():
        mss.ssd_chunk_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], chunk=Q, out=out, workspace=ws)

    ms = time_region(torch, step, args.steps, args.warmup)
    updates = b * L * H * P * N
    res = {"metric": "state updates/s (B*L*H*P*N), Mamba-2 SSD layer", "value": updates / (ms * 1e-3),
           "unit": "state updates/s", "ms_per_step": ms, "dtype": "bf16 MFMA operands, f32 accumulate",
           "config": {"workload": f"{cfg.name}: SSD b={b} L={L} H={H} P={P} G={G} N={N} chunk={Q}, bf16 x/B/C, "
                                  "fp32 delta/y/states", "batch": b, "seqlen": L, "nheads": H, "headdim": P,
                      "d_state": N, "chunk": Q}}
    if args.seqlen or args.batch:
        res["config"]["inputs"] = f"the preset's b={cfg.batch} L={cfg.seqlen} draw repeated or cut along b and L"
    cpu = None
    if not args.no_cpu_baseline and not (args.seqlen or args.batch):
        import oracle
        th, info = host_cpus()
        args64 = (I.to_f64(x["x"], "bf16"), x["delta"].astype(np.float64), x["A"], I.to_f64(x["B"], "bf16"),
                  I.to_f64(x["C"], "bf16"))
        h1 = 2  # one thread: batch row 0, heads 0..1
        one = (np.ascontiguousarray(args64[0][:1, :, :h1]), np.ascontiguousarray(args64[1][:1, :, :h1]),
               args64[2][:h1], args64[3][:1], args64[4][:1])
        cpu = cpu_leg(lambda: oracle.ssd(*args64, threads=th), b * L * H * P * N,
                      lambda: oracle.ssd(*one, threads=1), L * h1 * P * N, "state updates/s", th, info,
                      f"the whole workload (b={b}, L={L}, all heads)", f"batch row 0, heads 0..{h1 - 1}")
    res["mfma_flops"] = ssd_mfma_flops(b, L, H, P, N, Q)
    return res, ssd_bytes(b, L, H, P, G, N, 2), ms, "ssd kernels", ["ssd.hip", "ssd_common.hpp", "common.hpp"], cpu


def bench_ssd_bwd(args, torch, mss, I):
    cfg = I.SSD_2P8B
    x = I.ssd_inputs(cfg)
    x.update(I.ssd_grad_output(cfg))
    g = {k: to_dev(torch, x[k]) for k in ("x", "delta", "A", "B", "C", "dy")}
    b, L, H, P, G, N = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate
    ws = torch.empty(mss.ssd_bwd_workspace_size(b, L, H, P, G, N), dtype=torch.uint8, device="cuda:0")
    out = mss.ssd_chunk_bwd(g["x"], g["delta"], g["A"], g["B"], g["C"], dy=g["dy"], want_dD=False, want_dh0=False,
                            workspace=ws)

    def step():
        mss.ssd_chunk_bwd(g["x"], g["delta"], g["A"], g["B"], g["C"], dy=g["dy"], want_dD=False, want_dh0=False,
                          out=out, workspace=ws)

    ms = time_region(torch, step, args.steps, args.warmup)
    updates = b * L * H * P * N
    res = {"metric": "state updates/s (B*L*H*P*N), Mamba-2 SSD layer backward", "value": updates / (ms * 1e-3),
           "unit": "state updates/s", "ms_per_step": ms, "dtype": "bf16 MFMA operands (hi/lo pairs), f32 accumulate",
           "config": {"workload": f"{cfg.name}_bwd: SSD backward b={b} L={L} H={H} P={P} G={G} N={N}, gradients "
                                  "of x, delta, A, B, C from dy (fp32); bf16 x/B/C, fp32 delta/dy/gradients; the "
                                  "states recomputed by a forward pass inside the call", "batch": b, "seqlen": L,
                      "nheads": H, "headdim": P, "d_state": N}}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        th, info = host_cpus()
        f64 = lambda k: I.to_f64(x[k], "bf16")
        X, Bm, Cm, dl, dy = f64("x"), f64("B"), f64("C"), x["delta"].astype(np.float64), x["dy"].astype(np.float64)
        hs = 16  # all threads: both batch rows, heads 0..15 (the oracle runs one thread per (batch, head))
        units = min(th, b * hs)

        def call(nb, nh, t):
            return oracle.ssd_bwd(np.ascontiguousarray(X[:nb, :, :nh]), np.ascontiguousarray(dl[:nb, :, :nh]),
                                  x["A"][:nh], Bm[:nb], Cm[:nb], dy=np.ascontiguousarray(dy[:nb, :, :nh]), threads=t)
        cpu = cpu_leg(lambda: call(b, hs, units), b * L * hs * P * N, lambda: call(1, 2, 1), L * 2 * P * N,
                      "state updates/s", units, info, f"batch rows 0..{b - 1}, heads 0..{hs - 1}, full L={L}",
                      "batch row 0, heads 0..1, full L")
    res["mfma_flops"] = ssd_bwd_mfma_flops(b, L, H, P, N)
    files = ["ssd.hip", "ssd_bwd.hip", "ssd_common.hpp", "common.hpp"]
    return res, ssd_bwd_bytes(b, L, H, P, G, N, 2), ms, "ssd backward kernels (forward pass included)", files, cpu


def bench_copy(args, torch):
    n = 1 << 28  # 1 GiB of fp32
    a = torch.empty(n, dtype=torch.float32, device="cuda:0").fill_(1.0)
    c = torch.empty_like(a)
    ms = time_region(torch, lambda: c.copy_(a), args.steps, args.warmup)
    res = {"metric": "device copy GB/s (read + write)", "value": 2 * n * 4 / (ms * 1e-3) / 1e9, "unit": "GB/s",
           "ms_per_step": ms, "dtype": "f32", "config": {"workload": "copy: 1 GiB fp32 device-to-device"}}
    return res, 2 * n * 4, ms, "copy", [], None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (got --gpus {args.gpus}); "
              "the hot path shards over batch and channels with no communication", file=sys.stderr)
        sys.exit(2)
    if args.seqlen < 0 or args.batch < 0 or ((args.seqlen or args.batch) and
                                             args.workload in ("decode_2p8b", "copy", "scan_2p8b_fused",
                                                               "scan_2p8b_fused_bwd", "ssd_2p8b_bwd", "decode_m3")):
        print("bench.py: --seqlen and --batch take positive sizes and apply to the scan and SSD workloads",
              file=sys.stderr)
        sys.exit(2)
    if args.dstate < 0 or (args.dstate and args.workload not in SCAN_WORKLOADS):
        print("bench.py: --dstate takes a positive size and applies to " + ", ".join(SCAN_WORKLOADS), file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    sys.path.insert(0, ROOT)
    import selective_state_space_27_amd as mss
    from selective_state_space_27_amd import inputs as I

    def scan_cfg(cfg):
        if not args.dstate:
            return cfg
        return dataclasses.replace(cfg, name=f"{cfg.name}_n{args.dstate}", dstate=args.dstate)

    if args.workload == "scan_2p8b":
        res, nbytes, launch_ms, kernel, files, cpu = bench_scan(args, torch, mss, I, scan_cfg(I.SCAN_2P8B))
    elif args.workload == "scan_130m":
        res, nbytes, launch_ms, kernel, files, cpu = bench_scan(args, torch, mss, I, scan_cfg(I.SCAN_130M))
    elif args.workload == "decode_2p8b":
        res, nbytes, launch_ms, kernel, files, cpu = bench_decode(args, torch, mss, I)
    elif args.workload == "ssd_2p8b":
        res, nbytes, launch_ms, kernel, files, cpu = bench_ssd(args, torch, mss, I)
    elif args.workload == "ssd_2p8b_bwd":
        res, nbytes, launch_ms, kernel, files, cpu = bench_ssd_bwd(args, torch, mss, I)
    elif args.workload == "scan_m2shape":
        res, nbytes, launch_ms, kernel, files, cpu = bench_scan(args, torch, mss, I, I.SCAN_M2)
    elif args.workload == "scan_2p8b_bwd":
        res, nbytes, launch_ms, kernel, files, cpu = bench_scan_bwd(args, torch, mss, I, scan_cfg(I.SCAN_2P8B))
    elif args.workload == "scan_2p8b_fused_bwd":
        res, nbytes, launch_ms, kernel, files, cpu = bench_scan_fused_bwd(args, torch, mss, I, scan_cfg(I.SCAN_2P8B))
    elif args.workload == "scan_2p8b_fused":
        res, nbytes, launch_ms, kernel, files, cpu = bench_scan_fused(args, torch, mss, I, scan_cfg(I.SCAN_2P8B))
    elif args.workload == "decode_m3":
        res, nbytes, launch_ms, kernel, files, cpu = bench_decode_m3(args, torch, mss, I)
    else:
        res, nbytes, launch_ms, kernel, files, cpu = bench_copy(args, torch)

    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    # (counters were taken at the presets' shapes only)
    traffic = recorded_traffic(args.workload, files) if files and not (args.seqlen or args.batch or args.dstate) \
        else None
    hbm = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
           "traffic": traffic, "kernel": kernel, "algorithmic_bytes_per_launch": nbytes, "launch_ms": launch_ms}
    roofs = [hbm]
    if "alu_flops" in res:  # fp32 vector arithmetic
        a = res.pop("alu_flops") / (launch_ms * 1e-3) / 1e12
        roofs.append({"bound": "alu", "achieved": a, "peak": ALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": a / ALU_PEAK_TFLOPS, "traffic": traffic, "kernel": kernel,
                      "peak_with_packed_fp32": ALU_PEAK_PACKED_TFLOPS, "algorithmic_bytes_per_launch": nbytes,
                      "launch_ms": launch_ms})
    if "mfma_flops" in res:  # bf16 matrix cores
        m = res.pop("mfma_flops") / (launch_ms * 1e-3) / 1e12
        roofs.append({"bound": "mfma", "achieved": m, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": m / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic, "kernel": kernel,
                      "algorithmic_bytes_per_launch": nbytes, "launch_ms": launch_ms})
    # The roof the kernel runs closest to binds; the others are reported beside it.
    roofs.sort(key=lambda r: -r["frac"])
    roofline = dict(roofs[0])
    for r in roofs[1:]:
        roofline[r["bound"]] = {k: r[k] for k in ("achieved", "peak", "unit", "frac")}
    line = {
        "metric": res["metric"], "value": res["value"], "unit": res["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res["ms_per_step"], **STEP_TIMES, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": res["dtype"],
        "data": "synthetic (seeded generator, workload shapes)", "config": res["config"], "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
