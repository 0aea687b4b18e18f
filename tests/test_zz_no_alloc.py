"""mss_selective_scan_fwd_noalloc (the selective scan on the library's fixed
per-GPU scratch, for callers that cannot allocate) against
mss_selective_scan_fwd with a caller workspace, through the C ABI: two calls
in a row, the second on a smaller input, each compared with the workspace
call (bitwise: the same kernels in the same launch configuration) and
within the parity bar; the status word is cleared by each call."""
import ctypes

import numpy as np
import pytest
import torch

import selective_state_space_27_amd as mss
from selective_state_space_27_amd import inputs as I
from gpu_util import TOL, dev, host64, rel_err

pytestmark = pytest.mark.gpu

KEYS = ("u", "delta", "A", "B", "C", "D", "z")


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@pytest.mark.timeout(600)
def test_noalloc_matches_workspace_call_twice():
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda:0")
    # The headline layer shape (hand-offs between workgroups), then a smaller
    # single-sequence input whose pieces are cut along L (split passes).
    for cfg in (I.SCAN_2P8B, I.small_scan_config(1, 128, 16, 16384, "fp32", seed=I.SEED_BASE + 903)):
        x = I.scan_inputs(cfg, with_h0=True)
        g = {k: dev(x[k]) for k in KEYS}
        h0 = dev(x["h0"])
        b, d, n, L = cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen
        code = mss.MSS_BF16 if cfg.io == "bf16" else mss.MSS_FP32
        y = torch.empty_like(g["u"])
        hl = torch.empty((b, d, n), dtype=torch.float32, device="cuda:0")
        st = mss.lib().mss_selective_scan_fwd_noalloc(*(ptr(g[k]) for k in KEYS), ptr(h0), ptr(y), ptr(hl), b, d, n,
                                                      L, code, 0, ptr(status), stream)
        assert st == mss.MSS_OK, mss.lib().mss_status_string(st)
        yr, hr = mss.selective_scan_fwd(*(g[k] for k in KEYS), h0, return_last_state=True)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert torch.equal(y, yr) and torch.equal(hl, hr), cfg.name
        e1, e2 = rel_err(host64(y), host64(yr)), rel_err(host64(hl), host64(hr))
        assert e1 <= TOL[cfg.io] and e2 <= TOL[cfg.io]
        status.fill_(7)
        print(f"{cfg.name}: no-allocation call equals the workspace call (y {e1:.1e}, h_last {e2:.1e})")
