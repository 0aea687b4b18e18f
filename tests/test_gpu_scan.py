"""GPU parity of mss_selective_scan_fwd against the fp64 oracle.

Tolerance: max |g - r| / max(|r|, rms(r)) <= 1e-4 for fp32 I/O and 2e-2 for
bf16 I/O (bf16 outputs are rounded to nearest even; the oracle's are not).
The oracle receives exactly the inputs the GPU receives (bf16 widened
exactly).  Full-size workloads are compared on sampled channels, which the
oracle computes independently (channels do not interact).
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_27_amd as mss
from selective_state_space_27_amd import inputs as I
from gpu_util import assert_close, dev, host64, rel_err

pytestmark = pytest.mark.gpu


def run_gpu(x, force_general=False, with_h0=False, drop=()):
    io = x["io"]
    g = {k: (None if k in drop else dev(x[k])) for k in ("u", "delta", "A", "B", "C", "D", "z")}
    h0 = dev(x["h0"]) if with_h0 and x.get("h0") is not None else None
    y, hl = mss.selective_scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], h0,
                                   return_last_state=True, force_general_decay=force_general)
    torch.cuda.synchronize()
    return y, hl


def run_oracle(x, chans=None, with_h0=False, drop=()):
    io = x["io"]
    u, dl, z = I.to_f64(x["u"], io), I.to_f64(x["delta"], io), I.to_f64(x["z"], io)
    A, B, C, D = x["A"].astype(np.float64), I.to_f64(x["B"], io), I.to_f64(x["C"], io), x["D"].astype(np.float64)
    h0 = x["h0"].astype(np.float64) if with_h0 and x.get("h0") is not None else None
    if "D" in drop:
        D = None
    if "z" in drop:
        z = None
    if chans is None:
        return oracle.selective_scan(u, dl, A, B, C, D, z, h0)
    ys, hs = [], []
    for b, d in chans:   # one channel at a time: [1, 1, L]
        y, h = oracle.selective_scan(u[b:b + 1, d:d + 1], dl[b:b + 1, d:d + 1], A[d:d + 1], B[b:b + 1], C[b:b + 1],
                                     None if D is None else D[d:d + 1], None if z is None else z[b:b + 1, d:d + 1],
                                     None if h0 is None else h0[b:b + 1, d:d + 1])
        ys.append(y[0, 0])
        hs.append(h[0, 0])
    return np.stack(ys), np.stack(hs)


@pytest.mark.parametrize("force_general", [False, True])
def test_scan_tiny_workload(force_general):
    x = I.scan_inputs(I.SCAN_TINY)
    y, hl = run_gpu(x, force_general)
    ry, rh = run_oracle(x)
    print(f"tiny: y err {assert_close(host64(y), ry, 'fp32', 'y'):.2e}  h err {assert_close(host64(hl), rh, 'fp32', 'h_last'):.2e}")


SHAPES = [
    # b, d, N, L, io
    (1, 16, 16, 64, "fp32"),
    (2, 100, 16, 77, "fp32"),      # ragged channels and L (odd L: element loads)
    (2, 130, 4, 50, "bf16"),
    (1, 64, 1, 33, "fp32"),
    (2, 70, 64, 40, "fp32"),
    (1, 65, 64, 31, "bf16"),
    (3, 64, 12, 100, "bf16"),
    (1, 192, 16, 1, "fp32"),       # single step
    (2, 64, 16, 15, "bf16"),       # shorter than one tile
    (2, 64, 16, 300, "bf16"),      # several tiles and a ragged tail
    (1, 70, 128, 40, "fp32"),      # d_state 128: B/C loaded per 4-step block
    (2, 64, 100, 50, "bf16"),      # d_state 100: states past N padded with zeros
    (1, 130, 128, 33, "bf16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}d{}n{}l{}{}".format(*s))
@pytest.mark.parametrize("force_general", [False, True])
def test_scan_shapes_with_h0(shape, force_general):
    b, d, n, L, io = shape
    x = I.scan_inputs(I.small_scan_config(b, d, n, L, io), with_h0=True)
    y, hl = run_gpu(x, force_general, with_h0=True)
    ry, rh = run_oracle(x, with_h0=True)
    assert_close(host64(y), ry, io, "y")
    assert_close(host64(hl), rh, "fp32" if io == "fp32" else "bf16", "h_last")


@pytest.mark.parametrize("shape", [(2, 12800, 16, 45, "bf16"), (1, 16448, 16, 64, "fp32"), (3, 8200, 4, 37, "fp32")],
                         ids=lambda s: "b{}d{}n{}l{}{}".format(*s))
def test_scan_more_blocks_than_cus(shape):
    """More 64-channel blocks than compute units: the work is split evenly
    over one workgroup per CU, so sequences are cut mid-way and the state is
    handed from one workgroup to the next (ragged L, h0 and h_last included)."""
    b, d, n, L, io = shape
    x = I.scan_inputs(I.small_scan_config(b, d, n, L, io), with_h0=True)
    y, hl = run_gpu(x, with_h0=True)
    ry, rh = run_oracle(x, with_h0=True)
    assert_close(host64(y), ry, io, "y")
    assert_close(host64(hl), rh, "fp32" if io == "fp32" else "bf16", "h_last")
    y2, h2 = run_gpu(x, with_h0=True)
    assert torch.equal(y, y2) and torch.equal(hl, h2)


@pytest.mark.parametrize("drop", [("D",), ("z",), ("D", "z")])
def test_scan_optional_inputs(drop):
    x = I.scan_inputs(I.small_scan_config(2, 96, 16, 70, "fp32"))
    y, hl = run_gpu(x, drop=drop)
    ry, rh = run_oracle(x, drop=drop)
    assert_close(host64(y), ry, "fp32", "y")
    assert_close(host64(hl), rh, "fp32", "h_last")


def test_scan_general_a_matrix():
    """A without the S4D-real structure takes the per-state exp path."""
    x = I.scan_inputs(I.small_scan_config(2, 128, 16, 90, "fp32"))
    g = np.random.default_rng(3)
    x["A"] = (-np.exp(g.uniform(-1, 2, size=x["A"].shape))).astype(np.float32)
    x["A"][:64] = -(np.arange(16, dtype=np.float32) + 1)    # first block S4D, second general
    y, hl = run_gpu(x)
    ry, rh = run_oracle(x)
    assert_close(host64(y), ry, "fp32", "y")
    assert_close(host64(hl), rh, "fp32", "h_last")


@pytest.mark.parametrize("shape", [(2, 200, 16, 90, "fp32"), (1, 192, 128, 70, "bf16"), (2, 130, 128, 37, "fp32"),
                                   (1, 64, 1, 20, "fp32")],
                         ids=lambda s: "b{}d{}n{}l{}{}".format(*s))
def test_scan_decay_mode_per_block(shape):
    """Each 64-channel block takes its own decay path from A: A[d, n] equal
    over n (the Mamba-2 form, heads of 32 channels here), the S4D-real form,
    or neither; forcing the per-state path must agree."""
    b, d, n, L, io = shape
    x = I.scan_inputs(I.small_scan_config(b, d, n, L, io, a_form="head", head=32), with_h0=True)
    x["A"] = x["A"].copy()
    if d > 64:
        x["A"][64:128] = -0.5 * (np.arange(n, dtype=np.float32) + 1)       # S4D-real, A[d,0] = -0.5
    if d > 128:
        g = np.random.default_rng(5)
        x["A"][128:192] = -np.exp(g.uniform(-1.0, 1.5, size=x["A"][128:192].shape)).astype(np.float32)
    ry, rh = run_oracle(x, with_h0=True)
    hio = "fp32" if io == "fp32" else "bf16"
    for force in (False, True):
        y, hl = run_gpu(x, force, with_h0=True)
        assert_close(host64(y), ry, io, f"y force_general={force}")
        assert_close(host64(hl), rh, hio, f"h_last force_general={force}")


def test_scan_dstate128_more_blocks_than_cus():
    """d_state 128 with the sequence cut between workgroups (257 blocks)."""
    x = I.scan_inputs(I.small_scan_config(1, 16448, 128, 21, "bf16", a_form="head"), with_h0=True)
    y, hl = run_gpu(x, with_h0=True)
    ry, rh = run_oracle(x, with_h0=True)
    assert_close(host64(y), ry, "bf16", "y")
    assert_close(host64(hl), rh, "bf16", "h_last")


def test_scan_m2shape_workload_sampled():
    """The Mamba-1 scan on the SSD layer's shape (b=2, d_inner=5120 in 80
    heads, N=128, L=16384, bf16 I/O, A and delta shared within a head): the
    full launch, checked on 96 sampled channels."""
    x = I.scan_inputs(I.SCAN_M2)
    y, hl = run_gpu(x)
    g = np.random.default_rng(77)
    chans = [(int(b), int(d)) for b, d in zip(g.integers(0, 2, 96), g.integers(0, 5120, 96))]
    chans += [(0, 0), (1, 5119), (0, 64)]
    ry, rh = run_oracle(x, chans)
    yg, hg = host64(y), host64(hl)
    e1 = assert_close(np.stack([yg[b, d] for b, d in chans]), ry, "bf16", "y")
    gh = np.stack([hg[b, d] for b, d in chans])
    e2 = assert_close(gh, rh, "bf16", "h_last")
    assert rel_err(gh, rh) < 1e-4
    print(f"scan_m2shape sampled: y err {e1:.2e}  h_last err {e2:.2e}")


# Few sequences, long L: on a 256-CU part the scan cuts every sequence into
# pieces on all CUs (streams * 2 <= CUs and >= 8 tiles per piece) and runs the
# local pass, the carry chain and the final pass.
SPLIT_SHAPES = [
    # b, d, N, L, io, A form
    (1, 128, 16, 16384, "fp32", "s4d"),    # 2 streams over 256 workgroups: chains of 127 boundaries
    (2, 100, 16, 20001, "fp32", "s4d"),    # ragged channels and L (element loads)
    (1, 192, 128, 16384, "bf16", "head"),  # d_state 128, one decay for all states
    (1, 5120, 16, 4096, "bf16", "s4d"),    # the 2.8b layer at batch 1
]


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "b{}d{}n{}l{}{}_{}".format(*s))
def test_scan_split_along_l(shape):
    b, d, n, L, io, form = shape
    x = I.scan_inputs(I.small_scan_config(b, d, n, L, io, a_form=form), with_h0=True)
    ry, rh = run_oracle(x, with_h0=True)
    hio = "fp32" if io == "fp32" else "bf16"
    y, hl = run_gpu(x, with_h0=True)
    e1 = assert_close(host64(y), ry, io, "y")
    e2 = assert_close(host64(hl), rh, hio, "h_last")
    y2, h2 = run_gpu(x, with_h0=True)
    assert torch.equal(y, y2) and torch.equal(hl, h2)  # deterministic
    yg, hg = run_gpu(x, force_general=True, with_h0=True)
    assert_close(host64(yg), ry, io, "y (per-state exp)")
    assert_close(host64(hg), rh, hio, "h_last (per-state exp)")
    print(f"split {shape}: y err {e1:.2e}  h_last err {e2:.2e}")


@pytest.mark.timeout(900)
def test_scan_dstate128_arrangement_beyond_2p32_floats_sampled():
    """d_state 128 with batch*L >= 2^24: the fp32 B/C arrangement holds 2^32
    floats, more work-items than one dispatch can have, so its kernel loops
    over a capped grid.  b=1, d=64, L=2^24-5, fp32, inputs drawn on the
    device (seeded); three channels over the whole sequence against the
    oracle, and the call's status word."""
    L = (1 << 24) - 5
    cfg = I.small_scan_config(1, 64, 128, L, "fp32", seed=I.SEED_BASE + 902)
    g = I.scan_inputs_device(cfg)
    ws = torch.empty(mss.selective_scan_workspace_size(1, 64, 128, L, torch.float32), dtype=torch.uint8,
                     device="cuda:0")
    y, hl = mss.selective_scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                                   return_last_state=True, workspace=ws)
    assert mss.workspace_status(ws) == mss.MSS_OK
    chans = [0, 31, 63]
    h = lambda t: t.detach().cpu().numpy().astype(np.float64)
    ry, rh = oracle.selective_scan(h(g["u"][:, chans]), h(g["delta"][:, chans]), h(g["A"][chans]), h(g["B"]),
                                   h(g["C"]), h(g["D"][chans]), h(g["z"][:, chans]))
    e1 = assert_close(h(y[:, chans]), ry, "fp32", "y")
    e2 = assert_close(h(hl[:, chans]), rh, "fp32", "h_last")
    print(f"d_state 128, 2^32 arranged floats: y {e1:.2e} h_last {e2:.2e}")


def test_workspace_status_word():
    """The call's status word (the workspace's first 4 bytes): clear after a
    normal call with hand-offs between workgroups; a bounded wait that gives
    up sets it, here forced by writing the word from the host with a plain
    copy (no kernel is made to wait); the next call clears it."""
    x = I.scan_inputs(I.small_scan_config(2, 12800, 16, 45, "bf16"))
    g = {k: dev(x[k]) for k in ("u", "delta", "A", "B", "C", "D", "z")}
    ws = torch.empty(mss.selective_scan_workspace_size(2, 12800, 16, 45, torch.bfloat16), dtype=torch.uint8,
                     device="cuda:0")
    call = lambda **kw: mss.selective_scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                                               workspace=ws, **kw)
    y = call(check_waits=True)
    assert mss.workspace_status(ws) == mss.MSS_OK
    ws[:4].copy_(torch.tensor([1, 0, 0, 0], dtype=torch.uint8))
    assert mss.workspace_status(ws) == mss.MSS_ERR_WAIT
    with pytest.raises(mss.MambaScanError, match="MSS_ERR_WAIT"):
        mss._check_waits(ws, None, "forced")
    y2 = call(check_waits=True)
    assert mss.workspace_status(ws) == mss.MSS_OK
    assert torch.equal(y, y2)


def test_scan_split_general_a_and_long_sequence_sampled():
    """b=1, d_inner=5120, L=65536, bf16: a long single-sequence prefill, with
    one 64-channel block on a general A; checked on sampled channels."""
    x = I.scan_inputs(I.small_scan_config(1, 5120, 16, 65536, "bf16"))
    g = np.random.default_rng(11)
    x["A"] = x["A"].copy()
    x["A"][640:704] = -np.exp(g.uniform(-1.0, 1.5, size=(64, 16))).astype(np.float32)
    y, hl = run_gpu(x)
    chans = [(0, int(c)) for c in g.integers(0, 5120, 48)] + [(0, 0), (0, 640), (0, 703), (0, 5119)]
    ry, rh = run_oracle(x, chans)
    yg, hg = host64(y), host64(hl)
    assert_close(np.stack([yg[b, c] for b, c in chans]), ry, "bf16", "y")
    gh = np.stack([hg[b, c] for b, c in chans])
    assert_close(gh, rh, "bf16", "h_last")
    assert rel_err(gh, rh) < 1e-4


def test_scan_130m_workload_full():
    """b=8, d_inner=1536, N=16, L=2048, fp32: every output against the oracle."""
    x = I.scan_inputs(I.SCAN_130M)
    y, hl = run_gpu(x)
    ry, rh = run_oracle(x)
    e1 = assert_close(host64(y), ry, "fp32", "y")
    e2 = assert_close(host64(hl), rh, "fp32", "h_last")
    print(f"scan_130m: y err {e1:.2e}  h_last err {e2:.2e}")


@pytest.mark.timeout(900)
def test_scan_2p8b_workload_full():
    """b=4, d_inner=5120, N=16, L=8192, bf16 I/O (the headline launch): every
    element of y and h_last against the oracle."""
    x = I.scan_inputs(I.SCAN_2P8B)
    y, hl = run_gpu(x)
    yg, hg = host64(y), host64(hl)
    del y, hl
    ry, rh = run_oracle(x)
    e1 = assert_close(yg, ry, "bf16", "y")
    e2 = assert_close(hg, rh, "bf16", "h_last")
    # The state is never rounded to bf16: it meets the fp32 bar as well.
    e3 = rel_err(hg, rh)
    print(f"scan_2p8b full ({yg.size} outputs, {hg.size} states): y max rel err {e1:.3e}, "
          f"h_last {e2:.3e}; max abs err y {np.max(np.abs(yg - ry)):.3e}")
    assert e3 < 1e-4


def test_scan_deterministic_and_split_composition():
    """Bitwise run-to-run determinism; and scan(L) == scan(L1) then
    scan(L - L1, h0=h_last) bitwise (same arithmetic in the same order)."""
    x = I.scan_inputs(I.small_scan_config(2, 128, 16, 200, "bf16"))
    y1, h1 = run_gpu(x)
    y2, h2 = run_gpu(x)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    for L1 in (64, 37):
        a = dict(x)
        c = dict(x)
        for k in ("u", "delta", "B", "C", "z"):
            a[k] = np.ascontiguousarray(x[k][..., :L1])
            c[k] = np.ascontiguousarray(x[k][..., L1:])
        ya, ha = run_gpu(a)
        g = {k: dev(c[k]) for k in ("u", "delta", "A", "B", "C", "D", "z")}
        yc, hc = mss.selective_scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], ha,
                                        return_last_state=True)
        torch.cuda.synchronize()
        assert torch.equal(torch.cat([ya, yc], dim=2), y1), L1
        assert torch.equal(hc, h1), L1


def test_scan_causality_and_nan_propagation():
    x = I.scan_inputs(I.small_scan_config(1, 64, 16, 96, "fp32"))
    y, _ = run_gpu(x)
    for t0 in (0, 17, 95):
        x2 = dict(x)
        x2["u"] = x["u"].copy()
        x2["u"][0, 5, t0] += 2.0
        y2, _ = run_gpu(x2)
        assert torch.equal(y2[..., :t0], y[..., :t0])
        assert not torch.equal(y2[0, 5, t0], y[0, 5, t0])
    x3 = dict(x)
    x3["u"] = x["u"].copy()
    x3["u"][0, 9, 40] = np.nan
    y3, h3 = run_gpu(x3)
    y3 = y3.cpu()
    assert torch.isnan(y3[0, 9, 40:]).all() and not torch.isnan(y3[0, 9, :40]).any()
    others = torch.cat([y3[0, :9], y3[0, 10:]])
    assert not torch.isnan(others).any()
    assert torch.isnan(h3[0, 9]).all()


def test_scan_maximum_sizes_sampled():
    """At the documented limits: seqlen just under 2^24 and dim*seqlen just
    under 2^31, fp32 I/O (where a 64-channel block's rows come closest to the
    32-bit byte offsets), ragged L, two blocks for the whole chip (split
    passes).  Inputs drawn on the device (seeded); sampled channels over the
    whole sequence against the oracle."""
    L = (1 << 24) - 5
    cfg = I.small_scan_config(1, 128, 16, L, "fp32", seed=I.SEED_BASE + 900)
    g = I.scan_inputs_device(cfg)
    y, hl = mss.selective_scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                                   return_last_state=True)
    torch.cuda.synchronize()
    chans = [0, 77, 127]
    h = lambda t: t.detach().cpu().numpy().astype(np.float64)
    ry, rh = oracle.selective_scan(h(g["u"][:, chans]), h(g["delta"][:, chans]), h(g["A"][chans]), h(g["B"]),
                                   h(g["C"]), h(g["D"][chans]), h(g["z"][:, chans]))
    e1 = assert_close(h(y[:, chans]), ry, "fp32", "y")
    e2 = assert_close(h(hl[:, chans]), rh, "fp32", "h_last")
    print(f"maximum sizes: y {e1:.2e} h_last {e2:.2e}")
