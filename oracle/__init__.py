"""fp64 CPU oracle for the selective state space hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library never
imports, links or calls it, and the two share no code.

The arithmetic lives in ``mss_oracle.c`` (plain C, double precision, the
sequential recurrence exactly as the pages state it; see that file's header for
the passages and the readings taken).  This module only marshals numpy arrays
into it.  Inputs are widened exactly to fp64 by the caller (bf16 and fp32
values are representable in fp64).

Pins: every routine here is checked in ``tests/test_oracle_pins.py`` against
closed forms, library routines and brute force (time-invariant case equals a
causal convolution / first-order IIR filter, brute-force materialised matrix,
zero-input decay, chunk-split composition, scan equals repeated state updates,
SSD equals the Mamba-1 scan with scalar-per-head A and its matrix form, special
cases of D and the gate, linearity, causality; the scan prologue against a
library convolution and softplus's closed forms).
The backward is pinned by central finite differences of the forward, a
different computation.  The Mamba-3 step is pinned by its reduction to the
SSD recurrence (rank 1, real, Euler input), MIMO superposition over SSD runs,
the closed form of a rotating decaying state, the trapezoid rule's second-order
convergence on an ODE with a known solution, and the closed-form fixed point of
a constant input (real and complex).  The SSD backward is pinned by central
finite differences of the SSD forward and by its equality with the selective
scan's backward on the SSD's Mamba-1 form.  The fused scan's backward (numpy
here: the prologue's chain rule around the scan's backward) is pinned by
central finite differences of the fused forward.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_liboracle.so")
_SRC_PATH = os.path.join(_HERE, "mss_oracle.c")

_dp = ctypes.POINTER(ctypes.c_double)
_lib = None


def build_command() -> list[str]:
    """gcc command that builds the oracle's shared library (no fast-math)."""
    return ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-pthread",
            "-o", _LIB_PATH, _SRC_PATH, "-lm"]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"oracle library missing: {_LIB_PATH}; run __graft_entry__.build()")
        lib = ctypes.CDLL(_LIB_PATH)
        L = ctypes.c_long
        lib.oracle_selective_scan.argtypes = [_dp] * 10 + [L, L, L, L, ctypes.c_int]
        lib.oracle_selective_scan.restype = None
        lib.oracle_state_update.argtypes = [_dp] * 9 + [L, L, L, ctypes.c_int]
        lib.oracle_state_update.restype = None
        lib.oracle_ssd.argtypes = [_dp] * 11 + [L] * 7 + [ctypes.c_int]
        lib.oracle_ssd.restype = None
        lib.oracle_selective_scan_bwd.argtypes = [_dp] * 18 + [L, L, L, L, ctypes.c_int]
        lib.oracle_selective_scan_bwd.restype = None
        lib.oracle_scan_prologue.argtypes = [_dp] * 7 + [L, L, L, ctypes.c_int, ctypes.c_int]
        lib.oracle_scan_prologue.restype = None
        lib.oracle_ssd_bwd.argtypes = [_dp] * 18 + [L] * 6 + [ctypes.c_int]
        lib.oracle_ssd_bwd.restype = None
        lib.oracle_mamba3_step.argtypes = [_dp] * 12 + [L] * 6 + [ctypes.c_int, ctypes.c_int]
        lib.oracle_mamba3_step.restype = None
        _lib = lib
    return _lib


def _f64(a, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float64)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"oracle: expected shape {tuple(shape)}, got {a.shape}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def default_threads() -> int:
    """Threads the oracle uses: the CPUs this process may run on, at most 16."""
    env = os.environ.get("MSS_ORACLE_THREADS")
    if env:
        return max(1, int(env))
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def selective_scan(u, delta, A, B, C, D=None, z=None, h0=None, threads=None):
    """Plain sequential selective scan in fp64.

    u, delta, z: [b, d, L]; B, C: [b, N, L]; A: [d, N]; D: [d]; h0: [b, d, N].
    Returns (y [b, d, L], h_last [b, d, N]), both fp64.
    """
    u = _f64(u)
    b, d, L = u.shape
    N = np.shape(A)[1]
    delta = _f64(delta, (b, d, L))
    A = _f64(A, (d, N))
    B = _f64(B, (b, N, L))
    C = _f64(C, (b, N, L))
    D = _f64(D, (d,))
    z = _f64(z, (b, d, L))
    h0 = _f64(h0, (b, d, N))
    y = np.empty((b, d, L), dtype=np.float64)
    h_last = np.empty((b, d, N), dtype=np.float64)
    _load().oracle_selective_scan(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                  _ptr(h0), _ptr(y), _ptr(h_last), b, d, N, L,
                                  threads or default_threads())
    return y, h_last


def scan_prologue(x, conv_w, conv_b=None, delta_raw=None, delta_bias=None, conv_silu=False, softplus=True):
    """u and delta from the short causal convolution of x and the raw delta
    (see ``oracle_scan_prologue`` for the passages and readings).  x,
    delta_raw: [b, d, L]; conv_w: [d, 4]; conv_b, delta_bias: [d]."""
    x = _f64(x)
    b, d, L = x.shape
    w = _f64(conv_w, (d, 4))
    cb = None if conv_b is None else _f64(conv_b, (d,))
    dr = _f64(delta_raw, (b, d, L))
    db = None if delta_bias is None else _f64(delta_bias, (d,))
    u = np.empty((b, d, L))
    dl = np.empty((b, d, L))
    _load().oracle_scan_prologue(_ptr(x), _ptr(w), _ptr(cb), _ptr(dr), _ptr(db), _ptr(u), _ptr(dl), b, d, L,
                                 int(bool(conv_silu)), int(bool(softplus)))
    return u, dl


def selective_scan_fused(x, conv_w, conv_b, delta_raw, delta_bias, A, B, C, D=None, z=None, h0=None,
                         conv_silu=False, softplus=True, threads=None):
    """The scan fed by its prologue: u, delta = scan_prologue(...), then
    selective_scan(u, delta, ...).  Returns (y, h_last)."""
    u, dl = scan_prologue(x, conv_w, conv_b, delta_raw, delta_bias, conv_silu, softplus)
    return selective_scan(u, dl, A, B, C, D, z, h0, threads=threads)


def selective_scan_bwd(u, delta, A, B, C, D=None, z=None, h0=None, dy=None, dh_last=None, threads=None):
    """Gradient of a loss through the selective scan, in fp64 (mss_oracle.c,
    oracle_selective_scan_bwd): given dy = dloss/dy [b, d, L] and optionally
    dh_last = dloss/dh_last [b, d, N], returns a dict with du, ddelta [b, d, L],
    dA [d, N], dB, dC [b, N, L], dD [d] (None without D), dz [b, d, L] (None
    without z) and dh0 [b, d, N] (the gradient of the initial state)."""
    u = _f64(u)
    b, d, L = u.shape
    N = np.shape(A)[1]
    delta = _f64(delta, (b, d, L))
    A = _f64(A, (d, N))
    B = _f64(B, (b, N, L))
    C = _f64(C, (b, N, L))
    D = _f64(D, (d,))
    z = _f64(z, (b, d, L))
    h0 = _f64(h0, (b, d, N))
    dy = _f64(dy, (b, d, L))
    dh_last = _f64(dh_last, (b, d, N))
    g = {"du": np.empty((b, d, L)), "ddelta": np.empty((b, d, L)), "dA": np.empty((d, N)),
         "dB": np.empty((b, N, L)), "dC": np.empty((b, N, L)), "dD": np.empty(d) if D is not None else None,
         "dz": np.empty((b, d, L)) if z is not None else None, "dh0": np.empty((b, d, N))}
    _load().oracle_selective_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                      _ptr(dy), _ptr(dh_last), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]),
                                      _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]),
                                      b, d, N, L, threads or default_threads())
    return g


def selective_scan_fused_bwd(x, conv_w, conv_b, delta_raw, delta_bias, A, B, C, D=None, z=None, h0=None, dy=None,
                             dh_last=None, conv_silu=False, softplus=True, threads=None):
    """Gradient of a loss through selective_scan_fused, in fp64: the scan's
    gradient (selective_scan_bwd at u, delta = scan_prologue(...)) taken back
    through the prologue by the chain rule.  With c = conv_b + sum_k w_k
    x[t-3+k] (zeros before step 0) and v = delta_raw + delta_bias:
      dc = du * silu'(c) (du without silu),  silu'(c) = s (1 + c (1 - s)),
      s = 1 / (1 + exp(-c));  dv = ddelta * sigmoid(v) (ddelta without softplus);
      dx[s] = sum_k w_k dc[s + 3 - k] (terms past L dropped);
      dconv_w[:, k] = sum over batch and t of dc[t] x[t - 3 + k];
      dconv_b = sum of dc;  ddelta_raw = dv;  ddelta_bias = sum of dv.
    Returns the scan's dict (dA, dB, dC, dD, dz, dh0) with du and ddelta
    replaced by dx, ddelta_raw, dconv_w, dconv_b, ddelta_bias."""
    x = _f64(x)
    b, d, L = x.shape
    w = _f64(conv_w, (d, 4))
    cb = np.zeros(d) if conv_b is None else _f64(conv_b, (d,))
    dr = _f64(delta_raw, (b, d, L))
    dbias = np.zeros(d) if delta_bias is None else _f64(delta_bias, (d,))
    u, dl = scan_prologue(x, conv_w, conv_b, delta_raw, delta_bias, conv_silu, softplus)
    g = selective_scan_bwd(u, dl, A, B, C, D, z, h0, dy, dh_last, threads=threads)
    xp = np.concatenate([np.zeros((b, d, 3)), x], axis=2)  # xp[..., t + 3] = x[..., t]
    c = cb[None, :, None] + sum(w[None, :, k, None] * xp[:, :, k:k + L] for k in range(4))
    if conv_silu:
        s = 1.0 / (1.0 + np.exp(-c))
        dc = g["du"] * s * (1.0 + c * (1.0 - s))
    else:
        dc = g["du"]
    v = dr + dbias[None, :, None]
    dv = g["ddelta"] / (1.0 + np.exp(-v)) if softplus else g["ddelta"]
    dcp = np.concatenate([dc, np.zeros((b, d, 3))], axis=2)  # dcp[..., t] = dc[..., t], zero past L
    dx = sum(w[None, :, k, None] * dcp[:, :, 3 - k:3 - k + L] for k in range(4))
    dw = np.stack([np.sum(dc * xp[:, :, k:k + L], axis=(0, 2)) for k in range(4)], axis=1)
    out = dict(g)
    del out["du"], out["ddelta"]
    out.update({"dx": dx, "ddelta_raw": dv, "dconv_w": dw, "dconv_b": dc.sum(axis=(0, 2)),
                "ddelta_bias": dv.sum(axis=(0, 2))})
    return out


def state_update(h, u, delta, A, B, C, D=None, z=None, threads=None):
    """One recurrent step in fp64.  h: [b, d, N] (not modified; a new array is
    returned); u, delta, z: [b, d]; B, C: [b, N]; A: [d, N]; D: [d].
    Returns (h_new, y)."""
    h = np.array(h, dtype=np.float64, order="C", copy=True)
    b, d, N = h.shape
    u = _f64(u, (b, d))
    delta = _f64(delta, (b, d))
    A = _f64(A, (d, N))
    B = _f64(B, (b, N))
    C = _f64(C, (b, N))
    D = _f64(D, (d,))
    z = _f64(z, (b, d))
    y = np.empty((b, d), dtype=np.float64)
    _load().oracle_state_update(_ptr(h), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                _ptr(z), _ptr(y), b, d, N, threads or default_threads())
    return h, y


def ssd(x, delta, A, B, C, D=None, z=None, h0=None, chunk=None, threads=None):
    """Mamba-2 layer as its plain recurrence in fp64.

    x, z: [b, L, H, P]; delta: [b, L, H]; A, D: [H]; B, C: [b, L, G, N];
    h0: [b, H, P, N].  Returns (y [b, L, H, P], chunk_states or None, h_last).
    chunk_states [b, nchunks, H, P, N] is the state after the last step of each
    chunk of ``chunk`` steps (only when ``chunk`` is given).
    """
    x = _f64(x)
    b, L, H, P = x.shape
    G, N = np.shape(B)[2], np.shape(B)[3]
    delta = _f64(delta, (b, L, H))
    A = _f64(A, (H,))
    B = _f64(B, (b, L, G, N))
    C = _f64(C, (b, L, G, N))
    D = _f64(D, (H,))
    z = _f64(z, (b, L, H, P))
    h0 = _f64(h0, (b, H, P, N))
    if H % G:
        raise ValueError("nheads must be a multiple of ngroups")
    y = np.empty((b, L, H, P), dtype=np.float64)
    h_last = np.empty((b, H, P, N), dtype=np.float64)
    cs = None
    q = chunk if chunk else L
    if chunk:
        cs = np.empty((b, (L + chunk - 1) // chunk, H, P, N), dtype=np.float64)
    _load().oracle_ssd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                       _ptr(y), _ptr(cs), _ptr(h_last), b, L, H, P, G, N, q,
                       threads or default_threads())
    return y, cs, h_last


def ssd_bwd(x, delta, A, B, C, D=None, z=None, h0=None, dy=None, dh_last=None, threads=None):
    """Gradient of a loss through the SSD layer, in fp64 (mss_oracle.c,
    oracle_ssd_bwd): given dy = dloss/dy [b, L, H, P] and optionally dh_last
    [b, H, P, N], returns a dict with dx, dz (None without z) [b, L, H, P],
    ddelta [b, L, H], dA [H], dB, dC [b, L, G, N], dD [H] (None without D) and
    dh0 [b, H, P, N]."""
    x = _f64(x)
    b, L, H, P = x.shape
    G, N = np.shape(B)[2], np.shape(B)[3]
    delta = _f64(delta, (b, L, H))
    A = _f64(A, (H,))
    B = _f64(B, (b, L, G, N))
    C = _f64(C, (b, L, G, N))
    D = _f64(D, (H,))
    z = _f64(z, (b, L, H, P))
    h0 = _f64(h0, (b, H, P, N))
    dy = _f64(dy, (b, L, H, P))
    dh_last = _f64(dh_last, (b, H, P, N))
    g = {"dx": np.empty((b, L, H, P)), "ddelta": np.empty((b, L, H)), "dA": np.empty(H),
         "dB": np.empty((b, L, G, N)), "dC": np.empty((b, L, G, N)), "dD": np.empty(H) if D is not None else None,
         "dz": np.empty((b, L, H, P)) if z is not None else None, "dh0": np.empty((b, H, P, N))}
    _load().oracle_ssd_bwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(dy),
                           _ptr(dh_last), _ptr(g["dx"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]),
                           _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]), b, L, H, P, G, N,
                           threads or default_threads())
    return g


def mamba3_step(h, x, delta, A, B, C, D=None, z=None, x_prev=None, B_prev=None, theta=None, complex_state=False,
                threads=None):
    """One Mamba-3 generation step in fp64 (see ``oracle_mamba3_step`` in
    mss_oracle.c for the passages and the readings).  h: [b, H, P, N], or
    [b, H, P, N, 2] (re, im) when ``complex_state`` (not modified; a new array
    is returned); x, z, x_prev: [b, H, R, P]; B, C, B_prev: [b, G, R, N];
    delta: [b, H]; A, D: [H]; theta: [H, N].  x_prev and B_prev given = the
    trapezoid input rule.  Returns (h_new, y [b, H, R, P])."""
    h = np.array(h, dtype=np.float64, order="C", copy=True)
    x = _f64(x)
    b, H, R, P = x.shape
    N = np.shape(B)[3]
    G = np.shape(B)[1]
    if complex_state:
        if h.shape != (b, H, P, N, 2) or theta is None:
            raise ValueError("complex state: h is [b, H, P, N, 2] and theta [H, N] is required")
    elif h.shape != (b, H, P, N):
        raise ValueError("h must be [b, H, P, N]")
    if (x_prev is None) != (B_prev is None):
        raise ValueError("x_prev and B_prev go together (the trapezoid rule)")
    delta = _f64(delta, (b, H))
    A = _f64(A, (H,))
    B = _f64(B, (b, G, R, N))
    C = _f64(C, (b, G, R, N))
    D = _f64(D, (H,))
    z = _f64(z, (b, H, R, P))
    x_prev = _f64(x_prev, (b, H, R, P))
    B_prev = _f64(B_prev, (b, G, R, N))
    theta = _f64(theta, (H, N)) if complex_state else None
    y = np.empty((b, H, R, P), dtype=np.float64)
    _load().oracle_mamba3_step(_ptr(h), _ptr(x), _ptr(x_prev), _ptr(delta), _ptr(A), _ptr(theta), _ptr(B),
                               _ptr(B_prev), _ptr(C), _ptr(D), _ptr(z), _ptr(y), b, H, P, G, N, R,
                               int(bool(complex_state)), threads or default_threads())
    return h, y
