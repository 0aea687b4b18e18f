"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, and every validation error is returned on the host before
any HIP call (fake, never-dereferenced pointer values are used)."""
import ctypes
import os
import re
import subprocess

import pytest

import selective_state_space_27_amd as mss

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mambascan.h")

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS, ALIAS, WAIT = 0, 1, 2, 3, 4, 5, 6, 7, 9
FP32, BF16 = 0, 1

# Fake device addresses: 16-byte aligned, far apart, never dereferenced.
BASE = 0x7F0000000000
GB = 1 << 32


def P(i, off=0):
    return ctypes.c_void_p(BASE + i * GB + off)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mss_[a-z_0-9]+)\s*\(", text)))


def test_library_loads_and_exports_every_header_symbol():
    lib = mss.lib()
    declared = header_functions()
    assert set(declared) == set(mss.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", mss.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (mss_\w+)", out))
    assert set(declared) <= exported
    assert mss.abi_version() == 2


def test_status_strings():
    lib = mss.lib()
    for code, name in mss.STATUS_NAMES.items():
        assert lib.mss_status_string(code).decode().startswith(name)
    assert lib.mss_status_string(99).decode() == "unknown mss_status"


def scan_call(**kw):
    b, d, n, L = kw.pop("shape", (2, 64, 16, 128))
    io = kw.pop("io", BF16)
    ws_bytes = kw.pop("ws_bytes", mss.lib().mss_selective_scan_workspace_size(b, d, n, L, io, 0) or 1 << 20)
    args = dict(u=P(0), delta=P(1), A=P(2), B=P(3), C=P(4), D=P(5), z=P(6), h0=P(7), y=P(8), h_last=P(9),
                ws=P(10), flags=0)
    args.update(kw)
    return mss.lib().mss_selective_scan_fwd(args["u"], args["delta"], args["A"], args["B"], args["C"], args["D"],
                                            args["z"], args["h0"], args["y"], args["h_last"], b, d, n, L, io,
                                            args["flags"], args["ws"], ws_bytes, None)


def test_scan_validation_errors():
    assert scan_call(u=None) == NULL
    assert scan_call(y=None) == NULL
    assert scan_call(A=None) == NULL
    assert scan_call(shape=(0, 64, 16, 128)) == SHAPE
    assert scan_call(shape=(2, -1, 16, 128)) == SHAPE
    assert scan_call(shape=(2, 64, 16, 0)) == SHAPE
    assert scan_call(shape=(2, 1 << 20, 16, 1 << 12)) == SHAPE
    assert scan_call(shape=(1, 64, 16, 1 << 24)) == SHAPE         # seqlen at 2^24
    assert scan_call(shape=(1, 256, 16, 1 << 23)) == SHAPE        # dim*seqlen = 2^31, seqlen < 2^24
    assert scan_call(io=7) == DTYPE
    assert scan_call(shape=(2, 64, 129, 128)) == UNSUP
    assert scan_call(flags=0x80) == UNSUP
    assert scan_call(z=P(6, 2)) == ALIGN
    assert scan_call(h_last=P(9, 4)) == ALIGN
    assert scan_call(ws=None) == WS
    assert scan_call(ws_bytes=16) == WS
    assert scan_call(y=P(0, 256)) == ALIAS            # y inside u
    assert scan_call(h_last=P(8, 4096)) == ALIAS      # h_last inside y
    assert scan_call(h_last=P(10)) == ALIAS           # h_last on the workspace


def fused_call(**kw):
    b, d, n, L = kw.pop("shape", (2, 64, 16, 128))
    io = kw.pop("io", BF16)
    ws_bytes = kw.pop("ws_bytes", mss.lib().mss_selective_scan_workspace_size(b, d, n, L, io, 0) or 1 << 20)
    args = dict(x=P(0), conv_w=P(11), conv_b=P(12), delta_raw=P(1), delta_bias=P(13), A=P(2), B=P(3), C=P(4),
                D=P(5), z=P(6), h0=P(7), y=P(8), h_last=P(9), ws=P(10), flags=mss.MSS_FLAG_DELTA_SOFTPLUS)
    args.update(kw)
    return mss.lib().mss_selective_scan_fwd_fused(args["x"], args["conv_w"], args["conv_b"], args["delta_raw"],
                                                  args["delta_bias"], args["A"], args["B"], args["C"], args["D"],
                                                  args["z"], args["h0"], args["y"], args["h_last"], b, d, n, L, io,
                                                  args["flags"], args["ws"], ws_bytes, None)


def test_fused_scan_validation_errors():
    """Every error of the fused entry point comes back from the host checks
    (fake device pointers: nothing may be enqueued)."""
    assert fused_call(x=None) == NULL
    assert fused_call(conv_w=None) == NULL
    assert fused_call(delta_raw=None) == NULL
    assert fused_call(y=None) == NULL
    assert fused_call(shape=(2, 64, 16, 0)) == SHAPE
    assert fused_call(io=7) == DTYPE
    assert fused_call(shape=(2, 64, 129, 128)) == UNSUP
    assert fused_call(flags=0x80) == UNSUP
    assert fused_call(conv_w=P(11, 4)) == ALIGN
    assert fused_call(delta_bias=P(13, 8)) == ALIGN
    assert fused_call(ws=None) == WS
    assert fused_call(ws_bytes=16) == WS
    assert fused_call(y=P(0, 256)) == ALIAS           # y inside x
    assert fused_call(y=P(11)) == ALIAS               # y on the taps
    assert fused_call(h_last=P(13)) == ALIAS          # h_last on the delta bias
    assert fused_call(h_last=P(8, 4096)) == ALIAS     # h_last inside y


def bwd_call(**kw):
    b, d, n, L = kw.pop("shape", (2, 64, 16, 128))
    io = kw.pop("io", BF16)
    ws_bytes = kw.pop("ws_bytes", mss.lib().mss_selective_scan_bwd_workspace_size(b, d, n, L, io, 0) or 1 << 20)
    args = dict(u=P(0), delta=P(1), A=P(2), B=P(3), C=P(4), D=P(5), z=P(6), h0=P(7), dy=P(8), dh_last=P(9),
                du=P(10), ddelta=P(11), dA=P(12), dB=P(13), dC=P(14), dD=P(15), dz=P(16), dh0=P(17), ws=P(18),
                flags=0)
    args.update(kw)
    return mss.lib().mss_selective_scan_bwd(*(args[k] for k in ("u", "delta", "A", "B", "C", "D", "z", "h0", "dy",
                                                                "dh_last", "du", "ddelta", "dA", "dB", "dC", "dD",
                                                                "dz", "dh0")),
                                            b, d, n, L, io, args["flags"], args["ws"], ws_bytes, None)


def test_scan_bwd_validation_enqueues_nothing():
    """Every error is found on the host (fake device pointers, no GPU)."""
    assert bwd_call(u=None) == NULL
    assert bwd_call(dy=None) == NULL
    assert bwd_call(dB=None) == NULL
    assert bwd_call(dz=None) == NULL                  # z given without dz
    assert bwd_call(z=None) == NULL                   # dz given without z
    assert bwd_call(shape=(2, 64, 129, 128)) == UNSUP  # d_state above 128
    assert bwd_call(shape=(2, 64, 16, 0)) == SHAPE
    assert bwd_call(io=7) == DTYPE
    assert bwd_call(flags=0x80) == UNSUP
    assert bwd_call(dA=P(12, 4)) == ALIGN
    assert bwd_call(ws=None) == WS
    assert bwd_call(ws_bytes=16) == WS
    assert bwd_call(du=P(0, 256)) == ALIAS            # du inside u
    assert bwd_call(ddelta=P(10, 64)) == ALIAS        # two outputs overlap
    assert bwd_call(dh0=P(18)) == ALIAS               # output on the workspace
    lib = mss.lib()
    assert lib.mss_selective_scan_bwd_workspace_size(4, 5120, 16, 8192, BF16, 0) > \
        lib.mss_selective_scan_workspace_size(4, 5120, 16, 8192, BF16, 0)
    assert lib.mss_selective_scan_bwd_workspace_size(4, 5120, 32, 8192, BF16, 0) > \
        lib.mss_selective_scan_bwd_workspace_size(4, 5120, 16, 8192, BF16, 0)
    # Above 32 states: a 32-state backward's workspace reused by every slice,
    # plus fp32 copies of the [batch, dim, seqlen] tensors; the same for any
    # d_state from 33 to 128, none above.
    wide = lib.mss_selective_scan_bwd_workspace_size(4, 5120, 33, 8192, BF16, 0)
    assert wide > lib.mss_selective_scan_bwd_workspace_size(4, 5120, 32, 8192, BF16, 0) + 10 * 4 * 5120 * 8192 * 4
    assert lib.mss_selective_scan_bwd_workspace_size(4, 5120, 128, 8192, BF16, 0) == wide
    assert lib.mss_selective_scan_bwd_workspace_size(4, 5120, 129, 8192, BF16, 0) == 0


def test_scan_workspace_query():
    lib = mss.lib()
    assert lib.mss_selective_scan_workspace_size(4, 5120, 16, 8192, BF16, 0) > 0
    assert lib.mss_selective_scan_workspace_size(4, 5120, 129, 8192, BF16, 0) == 0
    assert lib.mss_selective_scan_workspace_size(0, 5120, 16, 8192, BF16, 0) == 0
    assert lib.mss_selective_scan_workspace_size(1, 16, 16, 64, 3, 0) == 0


def update_call(**kw):
    b, d, n = kw.pop("shape", (4, 64, 16))
    io = kw.pop("io", BF16)
    a = dict(h=P(0), u=P(1), delta=P(2), A=P(3), B=P(4), C=P(5), D=P(6), z=P(7), y=P(8), flags=0)
    a.update(kw)
    return mss.lib().mss_state_update(a["h"], a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["y"],
                                      b, d, n, io, a["flags"], None)


def test_state_update_validation_errors():
    assert update_call(h=None) == NULL
    assert update_call(B=None) == NULL
    assert update_call(shape=(4, 0, 16)) == SHAPE
    # At most 2^28 (batch, channel) rows: the grid stays below 2^31 work-items.
    assert update_call(shape=(1 << 8, 1 << 20, 16), flags=1) == UNSUP  # the shape passes; the flag is checked after it
    assert update_call(shape=(1 << 8, (1 << 20) + 1, 16)) == SHAPE
    assert update_call(shape=(1 << 14, 1 << 15, 128)) == SHAPE
    assert update_call(io=5) == DTYPE
    assert update_call(shape=(4, 64, 129)) == UNSUP
    assert update_call(flags=1) == UNSUP
    assert update_call(u=P(1, 8)) == ALIGN
    assert update_call(y=P(1, 16)) == ALIAS          # y overlaps u
    assert update_call(h=P(8)) == ALIAS              # h overlaps y
    assert update_call(h=P(3, 64)) == ALIAS          # h overlaps A


def ssd_call(**kw):
    b, L, H, Pd, G, N, Q = kw.pop("shape", (2, 1024, 8, 64, 1, 128, 256))
    io = kw.pop("io", BF16)
    ws_bytes = kw.pop("ws_bytes", mss.lib().mss_ssd_workspace_size(b, L, H, Pd, G, N, Q, io) or 1 << 20)
    a = dict(x=P(0), delta=P(1), A=P(2), B=P(3), C=P(4), D=P(5), z=P(6), h0=P(7), y=P(8), cs=P(9), hl=P(10),
             ws=P(11), flags=0)
    a.update(kw)
    return mss.lib().mss_ssd_chunk_fwd(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["h0"], a["y"],
                                       a["cs"], a["hl"], b, L, H, Pd, G, N, Q, io, a["flags"], a["ws"], ws_bytes,
                                       None)


def test_ssd_validation_errors():
    assert ssd_call(x=None) == NULL
    assert ssd_call(y=None) == NULL
    assert ssd_call(shape=(2, 0, 8, 64, 1, 128, 256)) == SHAPE
    assert ssd_call(io=9) == DTYPE
    assert ssd_call(io=FP32) == UNSUP
    assert ssd_call(shape=(2, 1024, 8, 32, 1, 128, 256)) == UNSUP     # headdim 32
    assert ssd_call(shape=(2, 1024, 8, 96, 1, 128, 256)) == UNSUP     # headdim 96
    assert ssd_call(shape=(2, 1024, 8, 64, 1, 40, 256)) == UNSUP      # dstate not a multiple of 16
    assert ssd_call(shape=(2, 1024, 8, 64, 1, 272, 256)) == UNSUP     # dstate above 256
    lib = mss.lib()
    for Pd, N in ((64, 16), (64, 48), (64, 64), (64, 128), (128, 128), (128, 64), (64, 192), (64, 256), (128, 256)):
        assert lib.mss_ssd_workspace_size(2, 1024, 8, Pd, 1, N, 256, BF16) > 0, (Pd, N)
    # headdim 128 runs as two 64-wide halves: twice the piece-state workspace.
    assert lib.mss_ssd_workspace_size(2, 1024, 8, 128, 1, 128, 256, BF16) > \
        lib.mss_ssd_workspace_size(2, 1024, 8, 64, 1, 128, 256, BF16)
    assert ssd_call(shape=(2, 1024, 8, 64, 1, 128, 100)) == UNSUP     # chunk
    assert ssd_call(shape=(2, 1024, 6, 64, 4, 128, 256)) == UNSUP     # nheads % ngroups
    # y's rows of one batch entry stay within 2^32 - 256 bytes: L*H*P <= 2^30 - 64.
    ws = lambda L, H, Pd=64: mss.lib().mss_ssd_workspace_size(1, L, H, Pd, 1, 128, 256, BF16)
    assert ws((1 << 16) - 1, 256) > 0
    assert ws(1 << 16, 256) == 0
    assert ws((1 << 15) - 1, 256, 128) > 0 and ws(1 << 15, 256, 128) == 0
    assert ws((1 << 24) - 1, 64) == 0 and ws(1 << 22, 64) == 0
    # Grids: chunks x 64-row head slices x batch below 2^22.
    assert mss.lib().mss_ssd_workspace_size(1024, 1024, 1024, 64, 1, 16, 64, BF16) == 0
    assert mss.lib().mss_ssd_workspace_size(1024, 1024, 255, 64, 1, 16, 64, BF16) > 0
    assert ssd_call(flags=2) == UNSUP
    assert ssd_call(B=P(3, 4)) == ALIGN
    assert ssd_call(ws=None) == WS
    assert ssd_call(ws_bytes=1) == WS
    assert ssd_call(y=P(0, 512)) == ALIAS
    assert ssd_call(hl=P(9)) == ALIAS                                  # h_last on chunk_states
    assert ssd_call(cs=P(11)) == ALIAS                                 # chunk_states on workspace


def ssd_bwd_call(**kw):
    b, L, H, Pd, G, N = kw.pop("shape", (2, 1024, 8, 64, 1, 128))
    io = kw.pop("io", BF16)
    ws_bytes = kw.pop("ws_bytes", mss.lib().mss_ssd_bwd_workspace_size(b, L, H, Pd, G, N, io) or 1 << 20)
    a = dict(x=P(0), delta=P(1), A=P(2), B=P(3), C=P(4), D=P(5), z=P(6), h0=P(7), dy=P(8), dhl=P(9), dx=P(10),
             ddelta=P(11), dA=P(12), dB=P(13), dC=P(14), dD=P(15), dz=P(16), dh0=P(17), ws=P(18), flags=0)
    a.update(kw)
    return mss.lib().mss_ssd_chunk_bwd(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["h0"], a["dy"],
                                       a["dhl"], a["dx"], a["ddelta"], a["dA"], a["dB"], a["dC"], a["dD"], a["dz"],
                                       a["dh0"], b, L, H, Pd, G, N, io, a["flags"], a["ws"], ws_bytes, None)


def test_ssd_bwd_validation_errors():
    """Everything rejected on the host before any HIP call (fake pointers)."""
    for k in ("x", "delta", "A", "B", "C", "dy", "dx", "ddelta", "dA", "dB", "dC"):
        assert ssd_bwd_call(**{k: None}) == NULL, k
    assert ssd_bwd_call(dz=None) == NULL                                 # z given without dz
    assert ssd_bwd_call(z=None) == NULL                                  # dz given without z
    assert ssd_bwd_call(shape=(2, 0, 8, 64, 1, 128)) == SHAPE
    assert ssd_bwd_call(io=9) == DTYPE
    assert ssd_bwd_call(io=FP32) == UNSUP
    assert ssd_bwd_call(shape=(2, 1024, 8, 96, 1, 128)) == UNSUP         # headdim 96
    assert ssd_bwd_call(shape=(2, 1024, 8, 64, 1, 40)) == UNSUP          # dstate not a multiple of 16
    assert ssd_bwd_call(shape=(2, 1024, 8, 64, 1, 272)) == UNSUP         # dstate above 256
    assert ssd_bwd_call(shape=(2, 1024, 6, 64, 4, 128)) == UNSUP         # nheads % ngroups
    lib = mss.lib()
    for Pd, N in ((64, 16), (64, 48), (64, 64), (64, 128), (128, 128), (128, 48)):
        assert lib.mss_ssd_bwd_workspace_size(2, 1024, 8, Pd, 1, N, BF16) > 0, (Pd, N)
    # Above 128 states: two halves, one d_state-128 workspace reused, plus
    # the half's B/C and state columns and the second half's sums.
    halves = lib.mss_ssd_bwd_workspace_size(2, 1024, 8, 64, 1, 256, BF16)
    assert halves > lib.mss_ssd_bwd_workspace_size(2, 1024, 8, 64, 1, 128, BF16)
    assert lib.mss_ssd_bwd_workspace_size(2, 1024, 8, 64, 1, 144, BF16) == halves
    assert lib.mss_ssd_bwd_workspace_size(2, 1024, 8, 64, 1, 272, BF16) == 0
    # The forward's limits with 64-step chunks: L*H*P below 2^30 - 64 and
    # ceil(L/64) * H * P/64 * batch below 2^22.
    assert lib.mss_ssd_bwd_workspace_size(1, (1 << 16) - 1, 256, 64, 1, 128, BF16) > 0
    assert lib.mss_ssd_bwd_workspace_size(1, 1 << 16, 256, 64, 1, 128, BF16) == 0
    assert lib.mss_ssd_bwd_workspace_size(64, 1 << 15, 128, 64, 1, 16, BF16) == 0
    assert ssd_bwd_call(flags=1) == UNSUP
    assert ssd_bwd_call(dy=P(8, 4)) == ALIGN
    assert ssd_bwd_call(ws=None) == WS
    assert ssd_bwd_call(ws_bytes=1) == WS
    assert ssd_bwd_call(dx=P(0, 512)) == ALIAS                           # dx over x
    assert ssd_bwd_call(dB=P(8)) == ALIAS                                # dB over dy
    assert ssd_bwd_call(dh0=P(10)) == ALIAS                              # dh0 over dx
    assert ssd_bwd_call(dC=P(18)) == ALIAS                               # dC over the workspace


def noalloc_call(**kw):
    b, d, n, L = kw.pop("shape", (2, 64, 16, 128))
    io = kw.pop("io", BF16)
    a = dict(u=P(0), delta=P(1), A=P(2), B=P(3), C=P(4), D=P(5), z=P(6), h0=P(7), y=P(8), h_last=P(9), st=P(10),
             flags=0)
    a.update(kw)
    return mss.lib().mss_selective_scan_fwd_noalloc(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                                    a["h0"], a["y"], a["h_last"], b, d, n, L, io, a["flags"], a["st"],
                                                    None)


def test_noalloc_validation_errors():
    """The no-allocation scan validates like the forward, plus its fixed
    scratch limit (64 MiB) and its status word, all before any HIP call."""
    lib = mss.lib()
    assert noalloc_call(u=None) == NULL
    assert noalloc_call(shape=(0, 64, 16, 128)) == SHAPE
    assert noalloc_call(shape=(2, 64, 129, 128)) == UNSUP
    assert noalloc_call(flags=0x8) == UNSUP
    assert noalloc_call(u=P(0, 8)) == ALIGN
    assert noalloc_call(st=P(10, 2)) == ALIGN          # the status word needs 4-byte alignment
    assert noalloc_call(y=P(0, 64)) == ALIAS
    assert noalloc_call(st=P(8, 64)) == ALIAS          # status word inside y
    assert noalloc_call(st=P(1, 4)) == ALIAS           # status word inside an input
    big = (4, 5120, 128, 8192)
    assert lib.mss_selective_scan_workspace_size(*big, BF16, 0) > mss.NOALLOC_SCRATCH_BYTES
    assert noalloc_call(shape=big) == WS
    assert lib.mss_selective_scan_workspace_size(4, 5120, 16, 8192, BF16, 0) < mss.NOALLOC_SCRATCH_BYTES


def test_workspace_status_rejects_null():
    assert mss.lib().mss_workspace_status(None, None) == NULL


def test_helper_grids_beyond_2p32_items_are_accepted():
    """The helper kernels loop over a capped grid, so shapes whose B/C
    arrangement or gradient sums exceed 2^32 elements are valid: d_state 128
    at batch*L >= 2^24 (2^32 arranged floats), and a backward whose dB, dC
    sums pass 2^32 elements."""
    lib = mss.lib()
    ws = lib.mss_selective_scan_workspace_size(1, 64, 128, (1 << 24) - 5, FP32, 0)
    assert ws > 4 * (1 << 32)
    assert lib.mss_selective_scan_workspace_size(4, 64, 128, (1 << 23) + 7, BF16, 0) > 0
    assert lib.mss_selective_scan_bwd_workspace_size(65535, 64, 32, 1 << 12, BF16, 0) > 0
    assert lib.mss_selective_scan_bwd_workspace_size(1, 64, 129, 1 << 12, BF16, 0) == 0  # d_state > 128


def test_python_binding_rejects_cpu_tensors():
    import torch
    u = torch.zeros(1, 16, 8)
    with pytest.raises(ValueError, match="GPU tensors only"):
        mss.selective_scan_fwd(u, u, torch.zeros(16, 4), torch.zeros(1, 4, 8), torch.zeros(1, 4, 8))


def m3_call(**kw):
    b, H, Pd, G, N, R = kw.pop("shape", (2, 4, 64, 2, 128, 4))
    io = kw.pop("io", BF16)
    a = dict(h=P(0), x=P(1), xp=P(2), delta=P(3), A=P(4), theta=P(5), B=P(6), Bp=P(7), C=P(8), D=P(9), z=P(10),
             y=P(11), flags=0x10)
    a.update(kw)
    return mss.lib().mss_mamba3_state_update(a["h"], a["x"], a["xp"], a["delta"], a["A"], a["theta"], a["B"],
                                             a["Bp"], a["C"], a["D"], a["z"], a["y"], b, H, Pd, G, N, R, io,
                                             a["flags"], None)


def test_mamba3_validation_errors():
    """Every error of the Mamba-3 step is found on the host (fake pointers);
    a call that passes every check is never made here."""
    assert m3_call(h=None) == NULL
    assert m3_call(xp=None) == NULL                   # x_prev without B_prev
    assert m3_call(Bp=None) == NULL
    assert m3_call(theta=None) == NULL                # complex state without theta
    assert m3_call(io=4) == DTYPE
    assert m3_call(shape=(2, 4, 0, 2, 128, 4)) == SHAPE
    assert m3_call(shape=(70000, 4, 64, 2, 128, 4)) == SHAPE
    assert m3_call(shape=(2, 4, 24, 2, 128, 4)) == UNSUP   # headdim not a multiple of 16
    assert m3_call(shape=(2, 4, 64, 2, 96, 4)) == UNSUP    # dstate not 64/128/256
    assert m3_call(shape=(2, 4, 64, 2, 128, 9)) == UNSUP   # rank above 8
    assert m3_call(shape=(2, 6, 64, 4, 128, 4)) == UNSUP   # nheads % ngroups
    assert m3_call(flags=0x11) == UNSUP
    assert m3_call(h=P(0, 8)) == ALIGN
    assert m3_call(y=P(1, 32)) == ALIAS                     # y on x
    assert m3_call(h=P(8, 64)) == ALIAS                     # state on C


def test_ssd_chunks_per_piece_override_and_workspace(monkeypatch):
    """MSS_SSD_CHUNKS_PER_PIECE sets the piece length of the SSD forward: more
    pieces need more piece-state workspace, the count stays at most 64, and
    a call whose workspace was sized under another setting that needs less
    is refused on the host (fake pointers; nothing is enqueued)."""
    shape = (2, 16384, 80, 64, 1, 128, 256)  # 64 chunks per sequence
    lib = mss.lib()
    monkeypatch.delenv("MSS_SSD_CHUNKS_PER_PIECE", raising=False)
    default = lib.mss_ssd_workspace_size(*shape, BF16)
    monkeypatch.setenv("MSS_SSD_CHUNKS_PER_PIECE", "64")  # one piece: no piece states beyond the first
    one = lib.mss_ssd_workspace_size(*shape, BF16)
    monkeypatch.setenv("MSS_SSD_CHUNKS_PER_PIECE", "1")   # 64 pieces, the most allowed
    many = lib.mss_ssd_workspace_size(*shape, BF16)
    assert one < default < many
    monkeypatch.setenv("MSS_SSD_CHUNKS_PER_PIECE", "0")   # not a positive count: the library's choice
    assert lib.mss_ssd_workspace_size(*shape, BF16) == default
    monkeypatch.setenv("MSS_SSD_CHUNKS_PER_PIECE", "1")
    assert ssd_call(shape=shape, ws_bytes=default) == WS  # sized for fewer pieces than the call now takes
    # At most 64 pieces: a shorter piece than 1/64 of the sequence is lengthened.
    long_shape = (1, 65536, 8, 64, 1, 128, 256)  # 256 chunks
    monkeypatch.setenv("MSS_SSD_CHUNKS_PER_PIECE", "4")
    cap = lib.mss_ssd_workspace_size(*long_shape, BF16)
    monkeypatch.setenv("MSS_SSD_CHUNKS_PER_PIECE", "1")
    assert lib.mss_ssd_workspace_size(*long_shape, BF16) == cap


def fused_bwd_call(**kw):
    b, d, n, L = kw.pop("shape", (2, 64, 16, 128))
    io = kw.pop("io", BF16)
    ws_bytes = kw.pop("ws_bytes", mss.lib().mss_selective_scan_fused_bwd_workspace_size(b, d, n, L, io, 0) or 1 << 20)
    names = ("x", "conv_w", "conv_b", "delta_raw", "delta_bias", "A", "B", "C", "D", "z", "h0", "dy", "dh_last", "dx",
             "ddelta_raw", "dconv_w", "dconv_b", "ddelta_bias", "dA", "dB", "dC", "dD", "dz", "dh0")
    args = {k: P(i) for i, k in enumerate(names)}
    args.update(ws=P(len(names)), flags=0)
    args.update(kw)
    return mss.lib().mss_selective_scan_fused_bwd(*(args[k] for k in names), b, d, n, L, io, args["flags"],
                                                  args["ws"], ws_bytes, None)


def test_fused_scan_bwd_validation_errors():
    """The fused backward's errors come back from the host checks (fake
    pointers; nothing is enqueued); its workspace covers the scan's backward
    and the fp32 copies, at any d_state the scan's backward takes."""
    for k in ("x", "conv_w", "delta_raw", "A", "B", "C", "dy", "dx", "ddelta_raw", "dconv_w", "dA", "dB", "dC"):
        assert fused_bwd_call(**{k: None}) == NULL, k
    assert fused_bwd_call(dz=None) == NULL              # z given without dz
    assert fused_bwd_call(z=None) == NULL               # dz given without z
    assert fused_bwd_call(shape=(2, 64, 16, 0)) == SHAPE
    assert fused_bwd_call(io=7) == DTYPE
    assert fused_bwd_call(shape=(2, 64, 129, 128)) == UNSUP
    assert fused_bwd_call(flags=0x80) == UNSUP
    assert fused_bwd_call(dconv_w=P(15, 4)) == ALIGN
    assert fused_bwd_call(ws=None) == WS
    assert fused_bwd_call(ws_bytes=16) == WS
    assert fused_bwd_call(dx=P(0, 256)) == ALIAS        # dx inside x
    assert fused_bwd_call(dconv_b=P(1)) == ALIAS        # dconv_b on the taps
    assert fused_bwd_call(ddelta_raw=P(13)) == ALIAS    # two outputs
    lib = mss.lib()
    for n in (16, 32, 64, 128):
        assert lib.mss_selective_scan_fused_bwd_workspace_size(4, 512, n, 1024, BF16, 0) > \
            lib.mss_selective_scan_bwd_workspace_size(4, 512, n, 1024, BF16, 0)
    assert lib.mss_selective_scan_fused_bwd_workspace_size(4, 512, 129, 1024, BF16, 0) == 0
