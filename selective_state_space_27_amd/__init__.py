"""Python binding of libmambascan (the MI355X selective state space hot path).

The functions here only marshal arguments into the C ABI declared in
``include/mambascan.h``: they check device/dtype/contiguity, allocate the
output and workspace tensors with PyTorch (device memory only) and pass raw
device pointers and the current HIP stream.  Every arithmetic step runs in the
library's HIP kernels.  There is no CPU fallback: if the library is missing
or a GPU is absent, the calls raise.

Operations (see the header for the exact definitions and layouts):
  selective_scan_fwd  Mamba-1 selective scan over a whole sequence
  selective_scan_fwd_noalloc  the same on the library's fixed per-GPU
                      scratch, for callers that cannot allocate
  selective_scan_fwd_fused  the same, fed by its prologue (short causal
                      convolution for u, delta from its raw value) in one pass
  selective_scan_bwd  its gradient
  state_update        one recurrent generation step, state updated in place
  mamba3_state_update one Mamba-3 generation step (trapezoid input, complex
                      state, MIMO rank R as options), state updated in place
  ssd_chunk_fwd       Mamba-2 SSD layer, chunked, dense products on MFMA
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmambascan.so")

MSS_OK = 0
MSS_FP32 = 0
MSS_BF16 = 1
MSS_FLAG_DECAY_GENERAL = 0x1
MSS_FLAG_CONV_SILU = 0x2
MSS_FLAG_DELTA_SOFTPLUS = 0x4
MSS_FLAG_COMPLEX_STATE = 0x10

STATUS_NAMES = {0: "MSS_OK", 1: "MSS_ERR_NULL", 2: "MSS_ERR_SHAPE", 3: "MSS_ERR_DTYPE", 4: "MSS_ERR_ALIGN",
                5: "MSS_ERR_UNSUPPORTED", 6: "MSS_ERR_WORKSPACE", 7: "MSS_ERR_ALIAS", 8: "MSS_ERR_HIP",
                9: "MSS_ERR_WAIT"}
MSS_ERR_WAIT = 9

# Every symbol the header declares.
EXPORTS = ("mss_selective_scan_fwd", "mss_selective_scan_fwd_noalloc", "mss_selective_scan_workspace_size",
           "mss_selective_scan_fwd_fused",
           "mss_selective_scan_bwd",
           "mss_selective_scan_bwd_workspace_size", "mss_selective_scan_fused_bwd",
           "mss_selective_scan_fused_bwd_workspace_size", "mss_state_update",
           "mss_mamba3_state_update",
           "mss_ssd_chunk_fwd", "mss_ssd_workspace_size", "mss_ssd_chunk_bwd", "mss_ssd_bwd_workspace_size",
           "mss_workspace_status", "mss_status_string",
           "mss_last_hip_error", "mss_abi_version")


class MambaScanError(RuntimeError):
    def __init__(self, status: int, what: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{what}: {lib().mss_status_string(status).decode()}"
        if status == 8:
            msg += f" (hipError_t {hip_error})"
        super().__init__(msg)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmambascan with argument types set (loads on first use)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libmambascan not built: {LIB_PATH} is missing "
                           "(run `python -m selective_state_space_27_amd.build`)")
    L = ctypes.CDLL(LIB_PATH)
    vp, fp, i64, u32, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    L.mss_selective_scan_fwd.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, vp, fp, i64, i64, i64, i64, ctypes.c_int,
                                         u32, vp, sz, vp]
    L.mss_selective_scan_fwd.restype = ctypes.c_int
    L.mss_selective_scan_fwd_noalloc.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, vp, fp, i64, i64, i64, i64,
                                                 ctypes.c_int, u32, vp, vp]
    L.mss_selective_scan_fwd_noalloc.restype = ctypes.c_int
    L.mss_selective_scan_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int, u32]
    L.mss_selective_scan_workspace_size.restype = sz
    L.mss_selective_scan_fwd_fused.argtypes = [vp, fp, fp, vp, fp, fp, vp, vp, fp, vp, fp, vp, fp, i64, i64, i64,
                                               i64, ctypes.c_int, u32, vp, sz, vp]
    L.mss_selective_scan_fwd_fused.restype = ctypes.c_int
    L.mss_selective_scan_bwd.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, vp, fp, vp, vp, fp, vp, vp, fp, vp, fp,
                                         i64, i64, i64, i64, ctypes.c_int, u32, vp, sz, vp]
    L.mss_selective_scan_bwd.restype = ctypes.c_int
    L.mss_selective_scan_bwd_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int, u32]
    L.mss_selective_scan_fused_bwd.argtypes = [vp] * 24 + [i64, i64, i64, i64, ctypes.c_int, u32, vp, sz, vp]
    L.mss_selective_scan_fused_bwd.restype = ctypes.c_int
    L.mss_selective_scan_fused_bwd_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int, u32]
    L.mss_selective_scan_fused_bwd_workspace_size.restype = sz
    L.mss_selective_scan_bwd_workspace_size.restype = sz
    L.mss_state_update.argtypes = [fp, vp, vp, fp, vp, vp, fp, vp, vp, i64, i64, i64, ctypes.c_int, u32, vp]
    L.mss_state_update.restype = ctypes.c_int
    L.mss_mamba3_state_update.argtypes = [vp, vp, vp, fp, fp, fp, vp, vp, vp, fp, vp, vp, i64, i64, i64, i64, i64,
                                          i64, ctypes.c_int, u32, vp]
    L.mss_mamba3_state_update.restype = ctypes.c_int
    L.mss_ssd_chunk_fwd.argtypes = [vp, fp, fp, vp, vp, fp, vp, fp, fp, fp, fp, i64, i64, i64, i64, i64, i64, i64,
                                    ctypes.c_int, u32, vp, sz, vp]
    L.mss_ssd_chunk_fwd.restype = ctypes.c_int
    L.mss_ssd_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, i64, ctypes.c_int]
    L.mss_ssd_workspace_size.restype = sz
    L.mss_ssd_chunk_bwd.argtypes = [vp, fp, fp, vp, vp, fp, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp, i64, i64,
                                    i64, i64, i64, i64, ctypes.c_int, u32, vp, sz, vp]
    L.mss_ssd_chunk_bwd.restype = ctypes.c_int
    L.mss_ssd_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int]
    L.mss_ssd_bwd_workspace_size.restype = sz
    L.mss_workspace_status.argtypes = [vp, vp]
    L.mss_workspace_status.restype = ctypes.c_int
    L.mss_status_string.argtypes = [ctypes.c_int]
    L.mss_status_string.restype = ctypes.c_char_p
    L.mss_last_hip_error.argtypes = []
    L.mss_last_hip_error.restype = ctypes.c_int
    L.mss_abi_version.argtypes = []
    L.mss_abi_version.restype = ctypes.c_int
    _lib = L
    return L


def abi_version() -> int:
    return lib().mss_abi_version()


# --------------------------------------------------------------- helpers ----
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _io_code(dtype) -> int:
    if dtype == torch.float32:
        return MSS_FP32
    if dtype == torch.bfloat16:
        return MSS_BF16
    raise TypeError(f"unsupported I/O dtype {dtype} (float32 or bfloat16)")


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _raise(status: int, what: str):
    if status != MSS_OK:
        raise MambaScanError(status, what, lib().mss_last_hip_error())


def _device_of(t: torch.Tensor) -> torch.device:
    if t.device.type != "cuda":
        raise ValueError("libmambascan works on GPU tensors only (no CPU path)")
    return t.device


def workspace_status(workspace, stream=None) -> int:
    """Waits for the stream, then reads the status word of the last call that
    used ``workspace`` (a uint8 device tensor): MSS_OK, or MSS_ERR_WAIT when a
    bounded wait between workgroups gave up and that call's outputs are not
    valid.  Other failures raise."""
    st = lib().mss_workspace_status(_ptr(workspace), _stream(stream))
    if st not in (MSS_OK, MSS_ERR_WAIT):
        _raise(st, "mss_workspace_status")
    return st


def _check_waits(workspace, stream, what):
    if workspace_status(workspace, stream) != MSS_OK:
        raise MambaScanError(MSS_ERR_WAIT, what)


# ------------------------------------------------------------ selective scan
def selective_scan_workspace_size(batch, dim, dstate, seqlen, dtype=torch.bfloat16, flags=0) -> int:
    return lib().mss_selective_scan_workspace_size(batch, dim, dstate, seqlen, _io_code(dtype), flags)


def selective_scan_fwd(u, delta, A, B, C, D=None, z=None, h0=None, *, return_last_state=False,
                       force_general_decay=False, out=None, h_last=None, workspace=None, stream=None,
                       check_waits=False):
    """Selective scan over the whole sequence.

    ``check_waits``: wait for the call and raise MambaScanError(MSS_ERR_WAIT)
    if a bounded wait between workgroups gave up (never expected; off by
    default because it synchronises).

    u, delta, z: [b, d, L]; B, C: [b, N, L] (float32 or bfloat16, all the same);
    A: [d, N] float32; D: [d] float32; h0: [b, d, N] float32.
    Returns y [b, d, L] (same dtype as u), and h_last [b, d, N] float32 when
    ``return_last_state``.
    """
    dev = _device_of(u)
    b, d, L = u.shape
    N = A.shape[1]
    io = u.dtype
    _check(u, "u", (b, d, L), io, dev)
    _check(delta, "delta", (b, d, L), io, dev)
    _check(A, "A", (d, N), torch.float32, dev)
    _check(B, "B", (b, N, L), io, dev)
    _check(C, "C", (b, N, L), io, dev)
    _check(D, "D", (d,), torch.float32, dev)
    _check(z, "z", (b, d, L), io, dev)
    _check(h0, "h0", (b, d, N), torch.float32, dev)
    flags = MSS_FLAG_DECAY_GENERAL if force_general_decay else 0
    code = _io_code(io)
    if out is None:
        out = torch.empty((b, d, L), dtype=io, device=dev)
    _check(out, "out", (b, d, L), io, dev)
    if return_last_state and h_last is None:
        h_last = torch.empty((b, d, N), dtype=torch.float32, device=dev)
    _check(h_last, "h_last", (b, d, N), torch.float32, dev)
    need = lib().mss_selective_scan_workspace_size(b, d, N, L, code, flags)
    if need == 0:
        _raise(5, "selective_scan_fwd")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib().mss_selective_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                      _ptr(out), _ptr(h_last), b, d, N, L, code, flags, _ptr(workspace),
                                      workspace.numel(), _stream(stream))
    _raise(st, "mss_selective_scan_fwd")
    if check_waits:
        _check_waits(workspace, stream, "mss_selective_scan_fwd")
    return (out, h_last) if return_last_state else out


NOALLOC_SCRATCH_BYTES = 64 << 20


def selective_scan_fwd_noalloc(u, delta, A, B, C, D=None, z=None, h0=None, *, return_last_state=False,
                               force_general_decay=False, out=None, h_last=None, wait_status=None, stream=None):
    """selective_scan_fwd on the library's fixed per-GPU scratch instead of a
    workspace (the library allocates nothing; ``out`` and ``h_last`` given
    make the call allocation-free here too).  Shapes that need more than
    NOALLOC_SCRATCH_BYTES of scratch raise MSS_ERR_WORKSPACE; calls that
    overlap in time on one GPU race.  ``wait_status``: an int32 device tensor
    of one element, set to 0, or nonzero if a bounded wait gave up."""
    dev = _device_of(u)
    b, d, L = u.shape
    N = A.shape[1]
    io = u.dtype
    _check(u, "u", (b, d, L), io, dev)
    _check(delta, "delta", (b, d, L), io, dev)
    _check(A, "A", (d, N), torch.float32, dev)
    _check(B, "B", (b, N, L), io, dev)
    _check(C, "C", (b, N, L), io, dev)
    _check(D, "D", (d,), torch.float32, dev)
    _check(z, "z", (b, d, L), io, dev)
    _check(h0, "h0", (b, d, N), torch.float32, dev)
    _check(wait_status, "wait_status", (1,), torch.int32, dev)
    if out is None:
        out = torch.empty((b, d, L), dtype=io, device=dev)
    _check(out, "out", (b, d, L), io, dev)
    if return_last_state and h_last is None:
        h_last = torch.empty((b, d, N), dtype=torch.float32, device=dev)
    _check(h_last, "h_last", (b, d, N), torch.float32, dev)
    flags = MSS_FLAG_DECAY_GENERAL if force_general_decay else 0
    st = lib().mss_selective_scan_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                              _ptr(h0), _ptr(out), _ptr(h_last), b, d, N, L, _io_code(io), flags,
                                              _ptr(wait_status), _stream(stream))
    _raise(st, "mss_selective_scan_fwd_noalloc")
    return (out, h_last) if return_last_state else out


def selective_scan_fwd_fused(x, conv_w, conv_b, delta_raw, delta_bias, A, B, C, D=None, z=None, h0=None, *,
                             conv_silu=False, softplus=True, return_last_state=False, force_general_decay=False,
                             out=None, h_last=None, workspace=None, stream=None, check_waits=False):
    """Selective scan whose u and delta are formed inside the kernel:
    u = conv_b + causal 4-tap depthwise convolution of x with conv_w (tap 3 on
    the current step), through silu if ``conv_silu``; delta = delta_raw +
    delta_bias, through softplus if ``softplus``.

    x, delta_raw, z: [b, d, L]; B, C: [b, N, L] (float32 or bfloat16, all the
    same); conv_w: [d, 4] float32; conv_b, delta_bias: [d] float32 or None;
    A, D, h0 as in selective_scan_fwd.  Returns y (and h_last) like it;
    ``check_waits`` as there."""
    dev = _device_of(x)
    b, d, L = x.shape
    N = A.shape[1]
    io = x.dtype
    _check(x, "x", (b, d, L), io, dev)
    _check(conv_w, "conv_w", (d, 4), torch.float32, dev)
    _check(conv_b, "conv_b", (d,), torch.float32, dev)
    _check(delta_raw, "delta_raw", (b, d, L), io, dev)
    _check(delta_bias, "delta_bias", (d,), torch.float32, dev)
    _check(A, "A", (d, N), torch.float32, dev)
    _check(B, "B", (b, N, L), io, dev)
    _check(C, "C", (b, N, L), io, dev)
    _check(D, "D", (d,), torch.float32, dev)
    _check(z, "z", (b, d, L), io, dev)
    _check(h0, "h0", (b, d, N), torch.float32, dev)
    flags = ((MSS_FLAG_DECAY_GENERAL if force_general_decay else 0) | (MSS_FLAG_CONV_SILU if conv_silu else 0) |
             (MSS_FLAG_DELTA_SOFTPLUS if softplus else 0))
    code = _io_code(io)
    if out is None:
        out = torch.empty((b, d, L), dtype=io, device=dev)
    _check(out, "out", (b, d, L), io, dev)
    if return_last_state and h_last is None:
        h_last = torch.empty((b, d, N), dtype=torch.float32, device=dev)
    _check(h_last, "h_last", (b, d, N), torch.float32, dev)
    need = lib().mss_selective_scan_workspace_size(b, d, N, L, code, flags)
    if need == 0:
        _raise(5, "selective_scan_fwd_fused")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib().mss_selective_scan_fwd_fused(_ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(delta_raw), _ptr(delta_bias),
                                            _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(out),
                                            _ptr(h_last), b, d, N, L, code, flags, _ptr(workspace), workspace.numel(),
                                            _stream(stream))
    _raise(st, "mss_selective_scan_fwd_fused")
    if check_waits:
        _check_waits(workspace, stream, "mss_selective_scan_fwd_fused")
    return (out, h_last) if return_last_state else out


def selective_scan_bwd_workspace_size(batch, dim, dstate, seqlen, dtype=torch.bfloat16, flags=0) -> int:
    return lib().mss_selective_scan_bwd_workspace_size(batch, dim, dstate, seqlen, _io_code(dtype), flags)


def selective_scan_bwd(u, delta, A, B, C, D=None, z=None, h0=None, *, dy, dh_last=None, want_dD=True,
                       want_dh0=False, force_general_decay=False, out=None, workspace=None, stream=None,
                       check_waits=False) -> dict:
    """Gradient of a loss through selective_scan_fwd (same inputs), given
    dy = dloss/dy [b, d, L] and optionally dh_last = dloss/dh_last [b, d, N]
    float32.  Returns a dict: du, ddelta, dz (None without z) [b, d, L] and dB,
    dC [b, N, L] in the I/O dtype; dA [d, N], dD [d] (None unless want_dD) and
    dh0 [b, d, N] (None unless want_dh0) in float32.  d_state <= 128.  ``out``:
    a dict from an earlier call with the same shapes whose tensors are
    written again (nothing is allocated for them).  ``check_waits`` as in
    selective_scan_fwd."""
    dev = _device_of(u)
    b, d, L = u.shape
    N = A.shape[1]
    io = u.dtype
    for t, name, shape, dt in ((u, "u", (b, d, L), io), (delta, "delta", (b, d, L), io), (A, "A", (d, N), torch.float32),
                               (B, "B", (b, N, L), io), (C, "C", (b, N, L), io), (D, "D", (d,), torch.float32),
                               (z, "z", (b, d, L), io), (h0, "h0", (b, d, N), torch.float32), (dy, "dy", (b, d, L), io),
                               (dh_last, "dh_last", (b, d, N), torch.float32)):
        _check(t, name, shape, dt, dev)
    flags = MSS_FLAG_DECAY_GENERAL if force_general_decay else 0
    code = _io_code(io)
    g = out if out is not None else {
         "du": torch.empty((b, d, L), dtype=io, device=dev), "ddelta": torch.empty((b, d, L), dtype=io, device=dev),
         "dA": torch.empty((d, N), dtype=torch.float32, device=dev),
         "dB": torch.empty((b, N, L), dtype=io, device=dev), "dC": torch.empty((b, N, L), dtype=io, device=dev),
         "dD": torch.empty((d,), dtype=torch.float32, device=dev) if want_dD else None,
         "dz": torch.empty((b, d, L), dtype=io, device=dev) if z is not None else None,
         "dh0": torch.empty((b, d, N), dtype=torch.float32, device=dev) if want_dh0 else None}
    for k, shape, dt in (("du", (b, d, L), io), ("ddelta", (b, d, L), io), ("dA", (d, N), torch.float32),
                         ("dB", (b, N, L), io), ("dC", (b, N, L), io), ("dD", (d,), torch.float32),
                         ("dz", (b, d, L), io), ("dh0", (b, d, N), torch.float32)):
        _check(g.get(k), k, shape, dt, dev)
    if (z is None) != (g.get("dz") is None):
        raise ValueError("dz is returned exactly when z is given")
    need = lib().mss_selective_scan_bwd_workspace_size(b, d, N, L, code, flags)
    if need == 0:
        _raise(5, "selective_scan_bwd")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib().mss_selective_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                      _ptr(dy), _ptr(dh_last), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]),
                                      _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g.get("dD")), _ptr(g.get("dz")),
                                      _ptr(g.get("dh0")),
                                      b, d, N, L, code, flags, _ptr(workspace), workspace.numel(), _stream(stream))
    _raise(st, "mss_selective_scan_bwd")
    if check_waits:
        _check_waits(workspace, stream, "mss_selective_scan_bwd")
    return g


def selective_scan_fused_bwd(x, conv_w, conv_b, delta_raw, delta_bias, A, B, C, D=None, z=None, h0=None, *, dy,
                             dh_last=None, conv_silu=False, softplus=True, want_dD=True, want_dh0=False,
                             force_general_decay=False, workspace=None, stream=None) -> dict:
    """Gradient of a loss through selective_scan_fwd_fused (same inputs and
    options), given dy [b, d, L] (I/O dtype) and optionally dh_last [b, d, N]
    float32.  Returns a dict: dx, ddelta_raw, dz (None without z) [b, d, L]
    and dB, dC [b, N, L] in the I/O dtype; dconv_w [d, 4], dconv_b and
    ddelta_bias [d] (None when the bias was None), dA [d, N], dD [d] (None
    unless want_dD) and dh0 [b, d, N] (None unless want_dh0) in float32."""
    dev = _device_of(x)
    b, d, L = x.shape
    N = A.shape[1]
    io = x.dtype
    f32 = torch.float32
    for t, name, shape, dt in ((x, "x", (b, d, L), io), (conv_w, "conv_w", (d, 4), f32), (conv_b, "conv_b", (d,), f32),
                               (delta_raw, "delta_raw", (b, d, L), io), (delta_bias, "delta_bias", (d,), f32),
                               (A, "A", (d, N), f32), (B, "B", (b, N, L), io), (C, "C", (b, N, L), io),
                               (D, "D", (d,), f32), (z, "z", (b, d, L), io), (h0, "h0", (b, d, N), f32),
                               (dy, "dy", (b, d, L), io), (dh_last, "dh_last", (b, d, N), f32)):
        _check(t, name, shape, dt, dev)
    flags = ((MSS_FLAG_DECAY_GENERAL if force_general_decay else 0) | (MSS_FLAG_CONV_SILU if conv_silu else 0) |
             (MSS_FLAG_DELTA_SOFTPLUS if softplus else 0))
    code = _io_code(io)
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
    g = {"dx": e((b, d, L), io), "ddelta_raw": e((b, d, L), io), "dconv_w": e((d, 4), f32),
         "dconv_b": e((d,), f32) if conv_b is not None else None,
         "ddelta_bias": e((d,), f32) if delta_bias is not None else None, "dA": e((d, N), f32),
         "dB": e((b, N, L), io), "dC": e((b, N, L), io), "dD": e((d,), f32) if want_dD else None,
         "dz": e((b, d, L), io) if z is not None else None, "dh0": e((b, d, N), f32) if want_dh0 else None}
    need = lib().mss_selective_scan_fused_bwd_workspace_size(b, d, N, L, code, flags)
    if need == 0:
        _raise(5, "selective_scan_fused_bwd")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib().mss_selective_scan_fused_bwd(
        _ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(delta_raw), _ptr(delta_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(z), _ptr(h0), _ptr(dy), _ptr(dh_last), _ptr(g["dx"]), _ptr(g["ddelta_raw"]), _ptr(g["dconv_w"]),
        _ptr(g["dconv_b"]), _ptr(g["ddelta_bias"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]),
        _ptr(g["dz"]), _ptr(g["dh0"]), b, d, N, L, code, flags, _ptr(workspace), workspace.numel(), _stream(stream))
    _raise(st, "mss_selective_scan_fused_bwd")
    return g


# -------------------------------------------------------------- state update
def state_update(h, u, delta, A, B, C, D=None, z=None, *, out=None, stream=None):
    """One generation step; ``h`` [b, d, N] float32 is updated in place.

    u, delta, z: [b, d]; B, C: [b, N] (float32 or bfloat16); A: [d, N];
    D: [d].  Returns y [b, d] in the I/O dtype."""
    dev = _device_of(h)
    b, d, N = h.shape
    io = u.dtype
    _check(h, "h", (b, d, N), torch.float32, dev)
    _check(u, "u", (b, d), io, dev)
    _check(delta, "delta", (b, d), io, dev)
    _check(A, "A", (d, N), torch.float32, dev)
    _check(B, "B", (b, N), io, dev)
    _check(C, "C", (b, N), io, dev)
    _check(D, "D", (d,), torch.float32, dev)
    _check(z, "z", (b, d), io, dev)
    if out is None:
        out = torch.empty((b, d), dtype=io, device=dev)
    _check(out, "out", (b, d), io, dev)
    st = lib().mss_state_update(_ptr(h), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                _ptr(out), b, d, N, _io_code(io), 0, _stream(stream))
    _raise(st, "mss_state_update")
    return out


# --------------------------------------------------------- Mamba-3 update
def mamba3_state_update(h, x, delta, A, B, C, D=None, z=None, *, x_prev=None, B_prev=None, theta=None, out=None,
                        stream=None):
    """One Mamba-3 generation step; ``h`` is updated in place.

    h: [b, H, P, N] float32, or [b, H, P, N, 2] (re, im) for the complex
    state, which needs theta [H, N] float32; x, z, x_prev: [b, H, R, P] and
    B, C, B_prev: [b, G, R, N] (float32 or bfloat16, all the same); delta:
    [b, H]; A, D: [H] float32.  x_prev and B_prev (the previous step's x and
    B) select the trapezoid input rule.  Returns y [b, H, R, P]."""
    dev = _device_of(h)
    b, H, R, P = x.shape
    G, N = B.shape[1], B.shape[3]
    io = x.dtype
    cplx = h.dim() == 5
    _check(h, "h", (b, H, P, N, 2) if cplx else (b, H, P, N), torch.float32, dev)
    if cplx and theta is None:
        raise ValueError("the complex state needs theta [H, N]")
    _check(x, "x", (b, H, R, P), io, dev)
    _check(x_prev, "x_prev", (b, H, R, P), io, dev)
    _check(delta, "delta", (b, H), torch.float32, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(theta, "theta", (H, N), torch.float32, dev)
    _check(B, "B", (b, G, R, N), io, dev)
    _check(B_prev, "B_prev", (b, G, R, N), io, dev)
    _check(C, "C", (b, G, R, N), io, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(z, "z", (b, H, R, P), io, dev)
    if out is None:
        out = torch.empty((b, H, R, P), dtype=io, device=dev)
    _check(out, "out", (b, H, R, P), io, dev)
    st = lib().mss_mamba3_state_update(_ptr(h), _ptr(x), _ptr(x_prev), _ptr(delta), _ptr(A),
                                       _ptr(theta if cplx else None), _ptr(B), _ptr(B_prev), _ptr(C), _ptr(D), _ptr(z),
                                       _ptr(out), b, H, P, G, N, R, _io_code(io),
                                       MSS_FLAG_COMPLEX_STATE if cplx else 0, _stream(stream))
    _raise(st, "mss_mamba3_state_update")
    return out


# ----------------------------------------------------------------------- SSD
def ssd_workspace_size(batch, seqlen, nheads, headdim, ngroups, dstate, chunk, dtype=torch.bfloat16) -> int:
    return lib().mss_ssd_workspace_size(batch, seqlen, nheads, headdim, ngroups, dstate, chunk, _io_code(dtype))


def ssd_chunk_fwd(x, delta, A, B, C, D=None, z=None, h0=None, *, chunk=256, return_chunk_states=False,
                  return_last_state=False, out=None, workspace=None, stream=None):
    """Mamba-2 SSD layer.

    x, z: [b, L, H, P] bfloat16; delta: [b, L, H] float32; A, D: [H] float32;
    B, C: [b, L, G, N] bfloat16; h0: [b, H, P, N] float32.
    Returns y [b, L, H, P] float32, plus chunk_states [b, nchunks, H, P, N]
    and/or h_last [b, H, P, N] when requested (in that order)."""
    dev = _device_of(x)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = x.dtype
    _check(x, "x", (b, L, H, P), io, dev)
    _check(delta, "delta", (b, L, H), torch.float32, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(B, "B", (b, L, G, N), io, dev)
    _check(C, "C", (b, L, G, N), io, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(z, "z", (b, L, H, P), io, dev)
    _check(h0, "h0", (b, H, P, N), torch.float32, dev)
    code = _io_code(io)
    nch = (L + chunk - 1) // chunk
    if out is None:
        out = torch.empty((b, L, H, P), dtype=torch.float32, device=dev)
    _check(out, "out", (b, L, H, P), torch.float32, dev)
    cs = torch.empty((b, nch, H, P, N), dtype=torch.float32, device=dev) if return_chunk_states else None
    hl = torch.empty((b, H, P, N), dtype=torch.float32, device=dev) if return_last_state else None
    need = lib().mss_ssd_workspace_size(b, L, H, P, G, N, chunk, code)
    if need == 0:
        _raise(5, "ssd_chunk_fwd")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib().mss_ssd_chunk_fwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                 _ptr(out), _ptr(cs), _ptr(hl), b, L, H, P, G, N, chunk, code, 0, _ptr(workspace),
                                 workspace.numel(), _stream(stream))
    _raise(st, "mss_ssd_chunk_fwd")
    res = [out]
    if return_chunk_states:
        res.append(cs)
    if return_last_state:
        res.append(hl)
    return res[0] if len(res) == 1 else tuple(res)


def ssd_bwd_workspace_size(batch, seqlen, nheads, headdim, ngroups, dstate, dtype=torch.bfloat16) -> int:
    return lib().mss_ssd_bwd_workspace_size(batch, seqlen, nheads, headdim, ngroups, dstate, _io_code(dtype))


def ssd_chunk_bwd(x, delta, A, B, C, D=None, z=None, h0=None, *, dy, dh_last=None, want_dD=True, want_dh0=True,
                  out=None, workspace=None, stream=None) -> dict:
    """Gradient of a loss through ssd_chunk_fwd (same inputs), given dy =
    dloss/dy [b, L, H, P] and optionally dh_last = dloss/dh_last [b, H, P, N],
    both float32.  Returns a dict of float32 tensors: dx, dz (None without z)
    [b, L, H, P], ddelta [b, L, H], dA [H], dB, dC [b, L, G, N], dD [H] (None
    unless want_dD) and dh0 [b, H, P, N] (None unless want_dh0).  d_state <=
    256.  ``out``: a dict from an earlier call with the same shapes whose
    tensors are written again."""
    dev = _device_of(x)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = x.dtype
    f32 = torch.float32
    for t, name, shape, dt in ((x, "x", (b, L, H, P), io), (delta, "delta", (b, L, H), f32), (A, "A", (H,), f32),
                               (B, "B", (b, L, G, N), io), (C, "C", (b, L, G, N), io), (D, "D", (H,), f32),
                               (z, "z", (b, L, H, P), io), (h0, "h0", (b, H, P, N), f32),
                               (dy, "dy", (b, L, H, P), f32), (dh_last, "dh_last", (b, H, P, N), f32)):
        _check(t, name, shape, dt, dev)
    code = _io_code(io)
    shapes = {"dx": (b, L, H, P), "ddelta": (b, L, H), "dA": (H,), "dB": (b, L, G, N), "dC": (b, L, G, N),
              "dD": (H,), "dz": (b, L, H, P), "dh0": (b, H, P, N)}
    want = {"dD": want_dD, "dz": z is not None, "dh0": want_dh0}
    g = out if out is not None else {
        k: (torch.empty(shp, dtype=f32, device=dev) if want.get(k, True) else None) for k, shp in shapes.items()}
    for k, shp in shapes.items():
        _check(g.get(k), k, shp, f32, dev)
    if (z is None) != (g.get("dz") is None):
        raise ValueError("dz is returned exactly when z is given")
    need = lib().mss_ssd_bwd_workspace_size(b, L, H, P, G, N, code)
    if need == 0:
        _raise(5, "ssd_chunk_bwd")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib().mss_ssd_chunk_bwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                 _ptr(dy), _ptr(dh_last), _ptr(g["dx"]), _ptr(g["ddelta"]), _ptr(g["dA"]),
                                 _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g.get("dD")), _ptr(g.get("dz")),
                                 _ptr(g.get("dh0")), b, L, H, P, G, N, code, 0, _ptr(workspace), workspace.numel(),
                                 _stream(stream))
    _raise(st, "mss_ssd_chunk_bwd")
    return g
