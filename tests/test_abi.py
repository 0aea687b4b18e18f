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

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS, ALIAS = 0, 1, 2, 3, 4, 5, 6, 7
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
    assert mss.abi_version() == 1


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
    assert bwd_call(shape=(2, 64, 33, 128)) == UNSUP  # d_state above 32
    assert bwd_call(shape=(65535, 1, 32, (1 << 24) - 1)) == SHAPE  # reduction grid beyond 2^31 blocks
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
    assert lib.mss_selective_scan_bwd_workspace_size(4, 5120, 33, 8192, BF16, 0) == 0


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
    assert ssd_call(shape=(2, 1024, 8, 32, 1, 128, 256)) == UNSUP     # headdim
    assert ssd_call(shape=(2, 1024, 8, 128, 1, 128, 256)) == UNSUP    # headdim 128 (64 only)
    assert ssd_call(shape=(2, 1024, 8, 64, 1, 256, 256)) == UNSUP     # dstate 256 (128 only)
    assert ssd_call(shape=(2, 1024, 8, 64, 1, 64, 256)) == UNSUP      # dstate
    assert ssd_call(shape=(2, 1024, 8, 64, 1, 128, 100)) == UNSUP     # chunk
    assert ssd_call(shape=(2, 1024, 6, 64, 4, 128, 256)) == UNSUP     # nheads % ngroups
    # y's rows of one batch entry stay within 2^32 - 256 bytes: L*H*P <= 2^30 - 64.
    ws = lambda L, H: mss.lib().mss_ssd_workspace_size(1, L, H, 64, 1, 128, 256, BF16)
    assert ws((1 << 16) - 1, 256) > 0
    assert ws(1 << 16, 256) == 0
    assert ws((1 << 24) - 1, 64) == 0 and ws(1 << 22, 64) == 0
    assert ssd_call(flags=2) == UNSUP
    assert ssd_call(B=P(3, 4)) == ALIGN
    assert ssd_call(ws=None) == WS
    assert ssd_call(ws_bytes=1) == WS
    assert ssd_call(y=P(0, 512)) == ALIAS
    assert ssd_call(hl=P(9)) == ALIAS                                  # h_last on chunk_states
    assert ssd_call(cs=P(11)) == ALIAS                                 # chunk_states on workspace


def test_python_binding_rejects_cpu_tensors():
    import torch
    u = torch.zeros(1, 16, 8)
    with pytest.raises(ValueError, match="GPU tensors only"):
        mss.selective_scan_fwd(u, u, torch.zeros(16, 4), torch.zeros(1, 4, 8), torch.zeros(1, 4, 8))
