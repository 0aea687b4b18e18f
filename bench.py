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
  scan_2p8b_fused  the headline scan fed by its prologue (u from the silu of
               the causal 4-tap convolution of x, delta = softplus(raw + bias))
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
METRIC = "state updates/s (B*L*D*N) + % HBM roofline, Mamba-2.8b-shaped scan"


SCAN_WORKLOADS = ("scan_2p8b", "scan_130m", "scan_2p8b_bwd", "scan_2p8b_fused")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="scan_2p8b",
                    choices=["scan_2p8b", "scan_130m", "decode_2p8b", "ssd_2p8b", "scan_m2shape", "scan_2p8b_bwd",
                             "scan_2p8b_fused", "copy"])
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


def time_region(torch, fn, steps, warmup):
    """Event-timed region on the current stream (the library launches there)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per step


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


def cpu_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


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
    files = ["scan.hip", "scan_layout.hpp", "common.hpp"]
    kernel = "scan_kernel (+ bc_transpose_kernel in the same timed call)"
    cpu = None
    if not args.no_cpu_baseline and not (args.seqlen or args.batch):
        import oracle
        f64 = lambda k: I.to_f64(x[k], cfg.io)  # the whole workload, repeated for at least CPU_MIN_S
        args64 = (f64("u"), f64("delta"), x["A"].astype(np.float64), f64("B"), f64("C"), x["D"].astype(np.float64),
                  f64("z"))
        th = cpu_threads()
        reps, dt = repeat_timed(lambda: oracle.selective_scan(*args64, threads=th))
        cpu = {"value": reps * b * d * n * L / dt, "unit": "state updates/s", "cores": th, "kind": "oracle",
               "sample": f"the whole workload (b={b}, d={d}, N={n}, L={L}) {reps} times; {dt:.2f} s wall, "
                         "fp64 C oracle"}
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
    files = ["scan.hip", "scan_layout.hpp", "common.hpp"]
    kernel = "scan_kernel with the fused prologue (+ bc_transpose_kernel in the same timed call)"
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        f64 = lambda k: I.to_f64(x[k], cfg.io)
        th = cpu_threads()
        call = lambda: oracle.selective_scan_fused(f64("x"), x["conv_w"], x["conv_b"], f64("delta_raw"),
                                                   x["delta_bias"], x["A"], f64("B"), f64("C"), x["D"], f64("z"),
                                                   conv_silu=True, softplus=True, threads=th)
        reps, dt = repeat_timed(call)
        cpu = {"value": reps * b * d * n * L / dt, "unit": "state updates/s", "cores": th, "kind": "oracle",
               "sample": f"the whole workload (b={b}, d={d}, N={n}, L={L}) {reps} times; {dt:.2f} s wall, "
                         "fp64 C oracle (prologue single-threaded, scan on the threads)"}
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
        th = cpu_threads()
        reps, dt = repeat_timed(lambda: oracle.selective_scan_bwd(*args64, threads=th))
        cpu = {"value": reps * d * n * L / dt, "unit": "state updates/s", "cores": th, "kind": "oracle",
               "sample": f"batch row 0 of {b} (all {d} channels, full L={L}) {reps} times; {dt:.2f} s wall, "
                         "fp64 C oracle backward"}
    files = ["scan.hip", "scan_bwd.hip", "scan_layout.hpp", "common.hpp"]
    kernel = "scan_bwd_kernel (+ checkpoint forward and bwd_reduce_kernel in the same timed call)"
    return res, scan_bwd_bytes(b, d, n, L, es), ms, kernel, files, cpu


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
        th = cpu_threads()

        def token_step():  # consecutive token steps over the whole batch, inputs cycling through the pool
            p = p64[state["s"] % I.DECODE_POOL]
            state["h"], _ = oracle.state_update(state["h"], p["u"], p["delta"], st["A"], p["B"], p["C"], st["D"],
                                                p["z"], threads=th)
            state["s"] += 1

        reps, dt = repeat_timed(token_step)
        cpu = {"value": b * d * n * reps / dt, "unit": "state updates/s", "cores": th, "kind": "oracle",
               "sample": f"all {b} batch rows, {reps} consecutive token steps; {dt:.2f} s wall"}
    # per-launch figures: one launch = one token step
    return res, nbytes, ms / cfg.steps, "state_update_kernel", ["state_update.hip", "common.hpp"], cpu


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
        th = cpu_threads()
        args64 = (I.to_f64(x["x"], "bf16"), x["delta"].astype(np.float64), x["A"], I.to_f64(x["B"], "bf16"),
                  I.to_f64(x["C"], "bf16"))
        reps, dt = repeat_timed(lambda: oracle.ssd(*args64, threads=th))
        cpu = {"value": reps * b * L * H * P * N / dt, "unit": "state updates/s", "cores": th, "kind": "oracle",
               "sample": f"the whole workload (b={b}, L={L}, all heads) {reps} times; {dt:.2f} s wall"}
    return res, ssd_bytes(b, L, H, P, G, N, 2), ms, "ssd kernels", ["ssd.hip", "common.hpp"], cpu


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
        print(f"bench.py: this build measures one GPU only (got --gpus {args.gpus}); "
              "the hot path shards over batch and channels with no communication", file=sys.stderr)
        sys.exit(2)
    if args.seqlen < 0 or args.batch < 0 or ((args.seqlen or args.batch) and
                                             args.workload in ("decode_2p8b", "copy", "scan_2p8b_fused")):
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
    elif args.workload == "scan_m2shape":
        res, nbytes, launch_ms, kernel, files, cpu = bench_scan(args, torch, mss, I, I.SCAN_M2)
    elif args.workload == "scan_2p8b_bwd":
        res, nbytes, launch_ms, kernel, files, cpu = bench_scan_bwd(args, torch, mss, I, scan_cfg(I.SCAN_2P8B))
    elif args.workload == "scan_2p8b_fused":
        res, nbytes, launch_ms, kernel, files, cpu = bench_scan_fused(args, torch, mss, I, scan_cfg(I.SCAN_2P8B))
    else:
        res, nbytes, launch_ms, kernel, files, cpu = bench_copy(args, torch)

    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    # (counters were taken at the presets' shapes only)
    traffic = recorded_traffic(args.workload, files) if files and not (args.seqlen or args.batch or args.dstate) \
        else None
    line = {
        "metric": res["metric"], "value": res["value"], "unit": res["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": res["dtype"], "data": "synthetic (seeded generator, workload shapes)",
        "config": res["config"],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": kernel,
                     "algorithmic_bytes_per_launch": nbytes, "launch_ms": launch_ms},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
