"""Seeded synthetic inputs for the selective-scan workloads.

This module is shared by the HIP path's tests/bench and by the fp64 oracle's
callers.  It holds input *preparation* only (random draws, the delta recipe,
bf16 rounding); none of the scan's own arithmetic lives here.

Workloads (shapes follow the Mamba pages: Mamba-1 blocks with d_state 16,
Mamba-2 blocks with d_state 128 and headdim 64, "Mamba State-Space Models"
skills page, usage section; the five workload shapes themselves are this
library's benchmark presets):

  scan_tiny     b=1  d_inner=16    N=16  L=64     fp32
  scan_130m     b=8  d_inner=1536  N=16  L=2048   fp32
  scan_2p8b     b=4  d_inner=5120  N=16  L=8192   bf16 I/O, fp32 A/D/state
  decode_2p8b   b=256 d_inner=5120 N=16  one token per step, 1000 steps
  ssd_2p8b      b=2  H=80 P=64 N=128 L=16384 chunk 256
  scan_m2shape  b=2  d_inner=5120 (80 heads of 64) N=128 L=16384, bf16 I/O,
                A and delta shared within a head (the Mamba-2 form)
  decode_m3     b=128 H=80 P=64 N=128 rank 4, one token per step: Mamba-3
                generation step with the trapezoid input rule and a complex
                (rotating) fp32 state, bf16 I/O (the Mamba-3 block example's
                d_state 128, headdim 64 and MIMO rank 4 at the 2.8b d_inner)

Every tensor comes from its own numpy PCG64 stream seeded by
SeedSequence([seed, tensor_id(, step)]), so the order in which tensors are
drawn cannot change their values.
"""
from __future__ import annotations

import dataclasses
import numpy as np

# Tensor ids for the per-tensor child streams.
TID_U, TID_DNOISE, TID_DT, TID_B, TID_C, TID_Z, TID_D, TID_H0, TID_A, TID_X, TID_DY, TID_CONVW, TID_CONVB = range(1, 14)
TID_THETA = 14
TID_DHL = 15

SEED_BASE = 27000


@dataclasses.dataclass(frozen=True)
class ScanConfig:
    name: str
    batch: int
    dim: int
    dstate: int
    seqlen: int
    io: str          # "fp32" or "bf16" (u, delta, B, C, z, y)
    seed: int
    # "s4d": A[d, n] = -(n+1) (the Mamba-1 S4D-real form), delta per channel.
    # "head": Mamba-2 form run through the Mamba-1 scan: channels in heads of
    #   `head` (a head's A[d, n] = A_h for every n, A_h = -exp(U(0, ln 16)) as
    #   in the SSD inputs, and one delta per (b, head, l) shared by its channels).
    a_form: str = "s4d"
    head: int = 64


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    dim: int
    dstate: int
    steps: int
    io: str          # dtype of u, delta, B, C, z, y; state h is always fp32
    seed: int


@dataclasses.dataclass(frozen=True)
class SSDConfig:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    chunk: int
    seed: int


SCAN_TINY = ScanConfig("scan_tiny", 1, 16, 16, 64, "fp32", SEED_BASE + 0)
SCAN_130M = ScanConfig("scan_130m", 8, 1536, 16, 2048, "fp32", SEED_BASE + 1)
SCAN_2P8B = ScanConfig("scan_2p8b", 4, 5120, 16, 8192, "bf16", SEED_BASE + 2)
DECODE_2P8B = DecodeConfig("decode_2p8b", 256, 5120, 16, 1000, "bf16", SEED_BASE + 3)
SSD_2P8B = SSDConfig("ssd_2p8b", 2, 16384, 80, 64, 1, 128, 256, SEED_BASE + 4)
@dataclasses.dataclass(frozen=True)
class Mamba3Config:
    name: str
    batch: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    rank: int
    steps: int
    io: str          # x, B, C, z, y; the state and delta, A, theta, D are fp32
    complex_state: bool
    trapezoid: bool
    seed: int


DECODE_M3 = Mamba3Config("decode_m3", 128, 80, 64, 1, 128, 4, 100, "bf16", True, True, SEED_BASE + 6)


# The Mamba-1 scan on the SSD workload's shape (d_inner = 80 heads x 64, N=128,
# the same b and L): the two kernels compared on one layer shape.
SCAN_M2 = ScanConfig("scan_m2shape", 2, 5120, 128, 16384, "bf16", SEED_BASE + 5, a_form="head")

# Distinct per-step input sets drawn for the 1000-step decode workload; step s
# uses set s % DECODE_POOL (the kernel's work does not depend on the values, and
# this keeps input generation and host memory bounded).
DECODE_POOL = 16


def rng(seed: int, tid: int, step: int | None = None) -> np.random.Generator:
    key = [int(seed), int(tid)] + ([int(step)] if step is not None else [])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


# ----------------------------------------------------------------- bf16 -----
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round fp32 values to bf16 with round-to-nearest-even; returns uint16 bits.

    NaN stays NaN (quiet); infinities and signed zeros are preserved."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = (bits + 0x7FFF + lsb) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = ((bits[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------- delta -----
def softplus(x: np.ndarray) -> np.ndarray:
    """Stable softplus in fp64: max(x,0) + log1p(exp(-|x|))."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def inv_softplus(y: np.ndarray) -> np.ndarray:
    """Inverse of softplus for y > 0: y + log(-expm1(-y))."""
    y = np.asarray(y, dtype=np.float64)
    return y + np.log(-np.expm1(-y))


def draw_dt(seed: int, count: int, lo: float = 1e-3, hi: float = 1e-1) -> np.ndarray:
    """dt log-uniform on [lo, hi], one per channel (or per head)."""
    g = rng(seed, TID_DT)
    return np.exp(g.uniform(np.log(lo), np.log(hi), size=count))


def make_delta(dt: np.ndarray, noise: np.ndarray, axis_shape) -> np.ndarray:
    """delta = softplus(0.5*noise + inv_softplus(dt)), computed in fp64.

    ``dt`` is broadcast against ``noise`` via ``axis_shape`` (a reshape of dt)."""
    return softplus(0.5 * noise.astype(np.float64) + inv_softplus(dt).reshape(axis_shape))


def _normal(seed, tid, shape, step=None) -> np.ndarray:
    return rng(seed, tid, step).standard_normal(size=shape, dtype=np.float32)


def _io(a: np.ndarray, io: str) -> np.ndarray:
    """fp32 array -> storage array for the I/O dtype (fp32 or uint16 bf16 bits)."""
    if io == "fp32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if io == "bf16":
        return f32_to_bf16_bits(a)
    raise ValueError(io)


def to_f64(a: np.ndarray, io: str) -> np.ndarray:
    """Exact widening of a storage array to fp64 (bf16 bits or fp32)."""
    if io == "bf16" or a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float64)


# ------------------------------------------------------------ scan inputs ---
def scan_inputs(cfg: ScanConfig, with_h0: bool = False) -> dict:
    """Inputs of the selective scan in storage form.

    u, delta, z: [b, d, l]; B, C: [b, n, l]  (I/O dtype)
    A: [d, n] fp32 = -(n+1) (S4D-real; a_form "head": A_h per head of channels);
    D: [d] fp32; h0: [b, d, n] fp32 (optional)
    """
    b, d, n, L, s = cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen, cfg.seed
    if cfg.a_form == "head":
        nh = -(-d // cfg.head)
        dt = draw_dt(s, nh)
        noise = _normal(s, TID_DNOISE, (b, nh, L))
        delta = make_delta(dt, noise, (1, nh, 1)).astype(np.float32)
        delta = np.ascontiguousarray(np.repeat(delta, cfg.head, axis=1)[:, :d])
        a_h = (-np.exp(rng(s, TID_A).uniform(0.0, np.log(16.0), size=nh))).astype(np.float32)
        A = np.ascontiguousarray(np.broadcast_to(np.repeat(a_h, cfg.head)[:d, None], (d, n)))
    else:
        dt = draw_dt(s, d)
        noise = _normal(s, TID_DNOISE, (b, d, L))
        delta = make_delta(dt, noise, (1, d, 1)).astype(np.float32)
        A = np.ascontiguousarray(np.broadcast_to(-(np.arange(n, dtype=np.float32) + 1.0), (d, n)))
    del noise
    out = {
        "u": _io(_normal(s, TID_U, (b, d, L)), cfg.io),
        "delta": _io(delta, cfg.io),
        "A": A,
        "B": _io(_normal(s, TID_B, (b, n, L)), cfg.io),
        "C": _io(_normal(s, TID_C, (b, n, L)), cfg.io),
        "D": _normal(s, TID_D, (d,)),
        "z": _io(_normal(s, TID_Z, (b, d, L)), cfg.io),
        "h0": (0.1 * _normal(s, TID_H0, (b, d, n))).astype(np.float32) if with_h0 else None,
        "io": cfg.io,
    }
    del delta
    return out


def scan_fused_inputs(cfg: ScanConfig, with_h0: bool = False) -> dict:
    """Inputs of the scan fed by its prologue, in storage form: the raw
    values whose short causal convolution and softplus give u and delta.

    x, delta_raw, z: [b, d, l] and B, C: [b, n, l] (I/O dtype); conv_w: [d, 4]
    ~ N(0, 0.5^2) and conv_b: [d] ~ N(0, 0.1^2) fp32; delta_raw = 0.5 N(0, 1)
    and delta_bias = inv_softplus(dt) per channel (dt log-uniform in
    [1e-3, 1e-1]), the workload's delta recipe before its softplus; A, D, h0
    as in scan_inputs (S4D-real A).
    """
    b, d, n, L, s = cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen, cfg.seed
    dt = draw_dt(s, d)
    return {
        "x": _io(_normal(s, TID_U, (b, d, L)), cfg.io),
        "conv_w": (0.5 * _normal(s, TID_CONVW, (d, 4))).astype(np.float32),
        "conv_b": (0.1 * _normal(s, TID_CONVB, (d,))).astype(np.float32),
        "delta_raw": _io((0.5 * _normal(s, TID_DNOISE, (b, d, L))).astype(np.float32), cfg.io),
        "delta_bias": inv_softplus(dt).astype(np.float32),
        "A": np.ascontiguousarray(np.broadcast_to(-(np.arange(n, dtype=np.float32) + 1.0), (d, n))),
        "B": _io(_normal(s, TID_B, (b, n, L)), cfg.io),
        "C": _io(_normal(s, TID_C, (b, n, L)), cfg.io),
        "D": _normal(s, TID_D, (d,)),
        "z": _io(_normal(s, TID_Z, (b, d, L)), cfg.io),
        "h0": (0.1 * _normal(s, TID_H0, (b, d, n))).astype(np.float32) if with_h0 else None,
        "io": cfg.io,
    }


def scan_inputs_device(cfg: ScanConfig, device="cuda:0") -> dict:
    """The scan_inputs distributions (S4D-real A) drawn on the device with
    torch's seeded generator, for sizes whose host draw would be too slow;
    fp32 I/O.  The values differ from scan_inputs' (another generator) but are
    as reproducible: same cfg, same tensors."""
    import torch
    b, d, n, L = cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed)
    kw = dict(generator=g, device=device, dtype=torch.float32)
    dt = torch.exp(torch.empty(d, device=device, dtype=torch.float64).uniform_(np.log(1e-3), np.log(1e-1), generator=g))
    bias = (dt + torch.log(-torch.expm1(-dt))).view(1, d, 1)  # inverse softplus
    delta = torch.empty((b, d, L), device=device, dtype=torch.float32)
    for i in range(b):  # softplus(0.5 eps + bias) per batch row, in fp64
        eps = torch.randn((d, L), **kw).double()
        delta[i] = torch.nn.functional.softplus(0.5 * eps + bias[0], threshold=40.0).float()
        del eps
    return {
        "u": torch.randn((b, d, L), **kw),
        "delta": delta,
        "A": -(torch.arange(n, device=device, dtype=torch.float32) + 1.0).repeat(d, 1),
        "B": torch.randn((b, n, L), **kw),
        "C": torch.randn((b, n, L), **kw),
        "D": torch.randn((d,), **kw),
        "z": torch.randn((b, d, L), **kw),
    }


def scan_grad_output(cfg: ScanConfig) -> np.ndarray:
    """dy = dloss/dy [b, d, l] ~ N(0, 1) in the I/O dtype, for the backward."""
    return _io(_normal(cfg.seed, TID_DY, (cfg.batch, cfg.dim, cfg.seqlen)), cfg.io)


# ---------------------------------------------------------- decode inputs ---
def decode_state0(cfg: DecodeConfig) -> np.ndarray:
    """Initial fp32 state h[b, d, n] ~ 0.1 * N(0, 1)."""
    return (0.1 * _normal(cfg.seed, TID_H0, (cfg.batch, cfg.dim, cfg.dstate))).astype(np.float32)


def decode_static(cfg: DecodeConfig) -> dict:
    """Per-layer parameters of the decode workload: A [d, n], D [d], dt [d]."""
    d, n = cfg.dim, cfg.dstate
    return {
        "A": np.ascontiguousarray(np.broadcast_to(-(np.arange(n, dtype=np.float32) + 1.0), (d, n))),
        "D": _normal(cfg.seed, TID_D, (d,)),
        "dt": draw_dt(cfg.seed, d),
    }


def decode_step_inputs(cfg: DecodeConfig, step: int, dt: np.ndarray) -> dict:
    """Fresh token inputs for one generation step (u, delta, z: [b, d]; B, C: [b, n])."""
    b, d, n, s = cfg.batch, cfg.dim, cfg.dstate, cfg.seed
    noise = _normal(s, TID_DNOISE, (b, d), step)
    delta = make_delta(dt, noise, (1, d)).astype(np.float32)
    return {
        "u": _io(_normal(s, TID_U, (b, d), step), cfg.io),
        "delta": _io(delta, cfg.io),
        "B": _io(_normal(s, TID_B, (b, n), step), cfg.io),
        "C": _io(_normal(s, TID_C, (b, n), step), cfg.io),
        "z": _io(_normal(s, TID_Z, (b, d), step), cfg.io),
        "io": cfg.io,
    }


# ------------------------------------------------------------- SSD inputs ---
def ssd_inputs(cfg: SSDConfig, with_h0: bool = False) -> dict:
    """Inputs of the SSD chunked layer.

    x: [b, l, h, p] bf16; B, C: [b, l, g, n] bf16; delta: [b, l, h] fp32;
    A: [h] fp32 = -exp(U(0, ln 16)); h0: [b, h, p, n] fp32 (optional).
    """
    b, L, H, P, G, N, s = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, cfg.seed
    dt = draw_dt(s, H)
    noise = _normal(s, TID_DNOISE, (b, L, H))
    delta = make_delta(dt, noise, (1, 1, H)).astype(np.float32)
    A = (-np.exp(rng(s, TID_A).uniform(0.0, np.log(16.0), size=H))).astype(np.float32)
    return {
        "x": f32_to_bf16_bits(_normal(s, TID_X, (b, L, H, P))),
        "delta": delta,
        "A": A,
        "B": f32_to_bf16_bits(_normal(s, TID_B, (b, L, G, N))),
        "C": f32_to_bf16_bits(_normal(s, TID_C, (b, L, G, N))),
        "h0": (0.1 * _normal(s, TID_H0, (b, H, P, N))).astype(np.float32) if with_h0 else None,
    }


def ssd_grad_output(cfg: SSDConfig, with_dh_last: bool = False) -> dict:
    """Loss gradients for the SSD backward: dy = dloss/dy [b, l, h, p] ~ N(0, 1)
    fp32 (the forward's output dtype) and dh_last = dloss/dh_last [b, h, p, n]
    ~ 0.1 N(0, 1) fp32 (optional)."""
    b, L, H, P, N, s = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.seed
    return {
        "dy": _normal(s, TID_DY, (b, L, H, P)),
        "dh_last": (0.1 * _normal(s, TID_DHL, (b, H, P, N))).astype(np.float32) if with_dh_last else None,
    }


def ssd_inputs_device(cfg: SSDConfig, device="cuda:0") -> dict:
    """The ssd_inputs distributions drawn on the device with torch's seeded
    generator (sizes whose host draw would be too slow): x, B, C bf16, delta
    and A fp32.  Reproducible per cfg; the values differ from ssd_inputs'."""
    import torch
    b, L, H, P, G, N = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed)
    kw = dict(generator=g, device=device, dtype=torch.float32)
    dt = torch.exp(torch.empty(H, device=device, dtype=torch.float64).uniform_(np.log(1e-3), np.log(1e-1), generator=g))
    bias = dt + torch.log(-torch.expm1(-dt))  # inverse softplus
    eps = torch.randn((b, L, H), **kw).double()
    delta = torch.nn.functional.softplus(0.5 * eps + bias, threshold=40.0).float()
    del eps
    A = -torch.exp(torch.empty(H, device=device, dtype=torch.float32).uniform_(0.0, float(np.log(16.0)), generator=g))
    return {
        "x": torch.randn((b, L, H, P), **kw).to(torch.bfloat16),
        "delta": delta,
        "A": A,
        "B": torch.randn((b, L, G, N), **kw).to(torch.bfloat16),
        "C": torch.randn((b, L, G, N), **kw).to(torch.bfloat16),
    }


# -------------------------------------------------------- Mamba-3 inputs ---
def mamba3_static(cfg: Mamba3Config) -> dict:
    """Per-layer parameters of a Mamba-3 decode workload: A [H] =
    -exp(U(0, ln 16)) and dt [H] (log-uniform on [1e-3, 1e-1]) as for SSD, D
    [H] ~ N(0, 1), theta [H, N] ~ U(-pi, pi) (rotation rate per state; the
    pages give no distribution), and the initial state 0.1 N(0, 1), [b, H, P,
    N] or [b, H, P, N, 2]."""
    b, H, P, N, s = cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, cfg.seed
    shape = (b, H, P, N, 2) if cfg.complex_state else (b, H, P, N)
    return {
        "A": (-np.exp(rng(s, TID_A).uniform(0.0, np.log(16.0), size=H))).astype(np.float32),
        "dt": draw_dt(s, H),
        "D": _normal(s, TID_D, (H,)),
        "theta": rng(s, TID_THETA).uniform(-np.pi, np.pi, size=(H, N)).astype(np.float32),
        "h0": (0.1 * _normal(s, TID_H0, shape)).astype(np.float32),
    }


def mamba3_step_inputs(cfg: Mamba3Config, step: int, dt: np.ndarray) -> dict:
    """Fresh token inputs of one Mamba-3 step: x, z [b, H, R, P] and B, C
    [b, G, R, N] ~ N(0, 1) in the I/O dtype; delta [b, H] fp32 from dt and
    per-element noise as in the other workloads."""
    b, H, P, G, N, R, s = cfg.batch, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, cfg.rank, cfg.seed
    noise = _normal(s, TID_DNOISE, (b, H), step)
    return {
        "x": _io(_normal(s, TID_X, (b, H, R, P), step), cfg.io),
        "B": _io(_normal(s, TID_B, (b, G, R, N), step), cfg.io),
        "C": _io(_normal(s, TID_C, (b, G, R, N), step), cfg.io),
        "z": _io(_normal(s, TID_Z, (b, H, R, P), step), cfg.io),
        "delta": make_delta(dt, noise, (1, H)).astype(np.float32),
    }


def small_mamba3_config(batch, nheads, headdim, ngroups, dstate, rank, steps, io="fp32", complex_state=True,
                        trapezoid=True, seed=SEED_BASE + 300) -> Mamba3Config:
    return Mamba3Config(f"m3_b{batch}_h{nheads}_p{headdim}_g{ngroups}_n{dstate}_r{rank}_{io}", batch, nheads, headdim,
                        ngroups, dstate, rank, steps, io, complex_state, trapezoid, seed)


def small_scan_config(batch, dim, dstate, seqlen, io="fp32", seed=SEED_BASE + 100, a_form="s4d",
                      head=64) -> ScanConfig:
    return ScanConfig(f"scan_b{batch}_d{dim}_n{dstate}_l{seqlen}_{io}_{a_form}", batch, dim, dstate, seqlen, io, seed,
                      a_form, head)


def small_ssd_config(batch, seqlen, nheads, headdim, ngroups, dstate, chunk, seed=SEED_BASE + 200) -> SSDConfig:
    return SSDConfig(f"ssd_b{batch}_l{seqlen}_h{nheads}_p{headdim}_g{ngroups}_n{dstate}_q{chunk}",
                     batch, seqlen, nheads, headdim, ngroups, dstate, chunk, seed)
