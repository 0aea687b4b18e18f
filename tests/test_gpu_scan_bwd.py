"""GPU parity of mss_selective_scan_bwd against the fp64 oracle backward.

The oracle's backward is pinned to central finite differences of its forward
(tests/test_oracle_pins.py).  Tolerance as for the forward: max |g - r| /
max(|r|, rms(r)) <= 1e-4 for fp32 I/O and 2e-2 for bf16 I/O (bf16 gradients
are rounded to nearest even).  dA and dD are always fp32.
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_27_amd as mss
from selective_state_space_27_amd import inputs as I
from gpu_util import assert_close, dev, host64, rel_err

pytestmark = pytest.mark.gpu


def grads_inputs(x, seed=99, with_dh_last=True):
    """dy (I/O dtype) and dh_last (fp32) for a loss through the scan."""
    b, d, L = x["u"].shape
    N = x["A"].shape[1]
    g = np.random.default_rng(seed)
    dy = g.standard_normal((b, d, L)).astype(np.float32)
    dy = I.f32_to_bf16_bits(dy) if x["io"] == "bf16" else dy
    dhl = (0.5 * g.standard_normal((b, d, N))).astype(np.float32) if with_dh_last else None
    return dy, dhl


def run_gpu_bwd(x, dy, dhl, drop=(), with_h0=True, force_general=False):
    g = {k: (None if k in drop else dev(x[k])) for k in ("u", "delta", "A", "B", "C", "D", "z")}
    h0 = dev(x["h0"]) if with_h0 and x.get("h0") is not None else None
    r = mss.selective_scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], h0, dy=dev(dy),
                               dh_last=dev(dhl), want_dD=True, want_dh0=True, force_general_decay=force_general)
    torch.cuda.synchronize()
    return {k: (None if v is None else host64(v)) for k, v in r.items()}


def run_oracle_bwd(x, dy, dhl, drop=(), with_h0=True, rows=None, chans=None):
    io = x["io"]
    sel = lambda a: a if rows is None else a[rows]
    u, dl, z = (sel(I.to_f64(x[k], io)) for k in ("u", "delta", "z"))
    B, C = sel(I.to_f64(x["B"], io)), sel(I.to_f64(x["C"], io))
    A, D = x["A"].astype(np.float64), x["D"].astype(np.float64)
    h0 = sel(x["h0"].astype(np.float64)) if with_h0 and x.get("h0") is not None else None
    dy64 = sel(I.to_f64(dy, io))
    dhl64 = None if dhl is None else sel(dhl.astype(np.float64))
    if "D" in drop:
        D = None
    if "z" in drop:
        z = None
    if chans is not None:  # a subset of channels (per-channel outputs and dA, dD only)
        u, dl, dy64 = u[:, chans], dl[:, chans], dy64[:, chans]
        z = None if z is None else z[:, chans]
        A, D = A[chans], None if D is None else D[chans]
        h0 = None if h0 is None else h0[:, chans]
        dhl64 = None if dhl64 is None else dhl64[:, chans]
    return oracle.selective_scan_bwd(u, dl, A, B, C, D, z, h0, dy64, dhl64)


def check(got, ref, io, keys=("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dh0")):
    errs = {}
    for k in keys:
        if ref.get(k) is None:
            assert got.get(k) is None or k == "dD", k
            continue
        tol_io = "fp32" if k in ("dA", "dD", "dh0") and io == "fp32" else io
        if k in ("dA", "dD", "dh0") and io == "bf16":
            tol_io = "bf16"  # computed from bf16-rounded inputs in fp32; compared at the bf16 bar
        errs[k] = assert_close(got[k], ref[k], tol_io, k)
    return errs


SHAPES = [
    # b, d, N, L, io
    (1, 16, 16, 64, "fp32"),
    (2, 100, 16, 77, "fp32"),      # ragged channels and L (element loads)
    (2, 130, 4, 50, "bf16"),
    (1, 64, 1, 33, "fp32"),        # one state per wave pair (SPW 1)
    (3, 64, 12, 100, "bf16"),      # states padded to the wave split
    (1, 192, 16, 1, "fp32"),       # single step
    (2, 64, 16, 15, "bf16"),       # shorter than one tile
    (2, 64, 16, 300, "bf16"),      # several tiles and a ragged tail
    (2, 100, 32, 77, "fp32"),      # 4 states per wave, ragged channels and L
    (2, 64, 24, 300, "bf16"),      # 4 states per wave, states padded
    (1, 128, 17, 40, "fp32"),      # one state above 16
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}d{}n{}l{}{}".format(*s))
def test_scan_bwd_shapes(shape):
    b, d, n, L, io = shape
    x = I.scan_inputs(I.small_scan_config(b, d, n, L, io), with_h0=True)
    dy, dhl = grads_inputs(x)
    got = run_gpu_bwd(x, dy, dhl)
    errs = check(got, run_oracle_bwd(x, dy, dhl), io)
    print(shape, {k: f"{v:.1e}" for k, v in errs.items()})


@pytest.mark.parametrize("drop", [("D",), ("z",), ("D", "z")])
def test_scan_bwd_optional_inputs(drop):
    x = I.scan_inputs(I.small_scan_config(2, 96, 16, 70, "fp32"))
    dy, _ = grads_inputs(x, with_dh_last=False)
    got = run_gpu_bwd(x, dy, None, drop=drop, with_h0=False)
    ref = run_oracle_bwd(x, dy, None, drop=drop, with_h0=False)
    if "D" in drop:  # the gradient at D = 0 is still returned when asked for
        ref_d = run_oracle_bwd(dict(x, D=np.zeros_like(x["D"])), dy, None, drop=tuple(k for k in drop if k != "D"),
                               with_h0=False)
        ref["dD"] = ref_d["dD"]
    check(got, ref, "fp32")


@pytest.mark.parametrize("n", [16, 32])
@pytest.mark.parametrize("force_general", [False, True])
def test_scan_bwd_general_a(force_general, n):
    x = I.scan_inputs(I.small_scan_config(2, 128, n, 90, "fp32"), with_h0=True)
    g = np.random.default_rng(3)
    x["A"] = (-np.exp(g.uniform(-1, 2, size=x["A"].shape))).astype(np.float32)
    x["A"][:64] = -(np.arange(n, dtype=np.float32) + 1)
    dy, dhl = grads_inputs(x)
    check(run_gpu_bwd(x, dy, dhl, force_general=force_general), run_oracle_bwd(x, dy, dhl), "fp32")


@pytest.mark.parametrize("shape", [(2, 12800, 16, 45, "bf16"), (1, 128, 16, 16384, "fp32"),
                                   (1, 5120, 16, 4096, "bf16"), (2, 100, 16, 20001, "fp32"),
                                   (1, 64, 4, 9000, "fp32"), (2, 10240, 16, 257, "bf16"),
                                   (2, 12800, 32, 45, "bf16"), (1, 128, 32, 9000, "fp32")],
                         ids=["carry_handoff", "split_passes", "split_b1_layer", "split_ragged", "split_spw1",
                              "split_two_pieces_per_range", "carry_handoff_n32", "split_passes_n32"])
def test_scan_bwd_checkpoint_paths(shape):
    """More streams than CUs (the backward's gradient and the forward's state
    handed between workgroups), and few long sequences (both cut over all CUs:
    the forward's split passes, and the backward's local adjoint pass, chain
    and final pass with per-workgroup partial sums)."""
    b, d, n, L, io = shape
    x = I.scan_inputs(I.small_scan_config(b, d, n, L, io), with_h0=True)
    dy, dhl = grads_inputs(x)
    errs = check(run_gpu_bwd(x, dy, dhl), run_oracle_bwd(x, dy, dhl), io)
    print(shape, {k: f"{v:.1e}" for k, v in errs.items()})


WIDE_SHAPES = [
    # b, d, N, L, io: d_state above 32, taken by slices of 32 states
    (2, 100, 40, 77, "fp32"),      # slices of 32 and 8, ragged channels and L
    (1, 64, 64, 150, "fp32"),      # two full slices
    (2, 80, 128, 60, "bf16"),      # four slices, bf16 I/O (fp32 inside, rounded once)
    (1, 130, 33, 40, "fp32"),      # a one-state last slice
    (1, 33, 40, 31, "bf16"),       # b*d*L not a multiple of 4 (partial last group of the flat passes)
    (1, 35, 48, 29, "fp32"),
]


@pytest.mark.parametrize("shape", WIDE_SHAPES, ids=lambda s: "b{}d{}n{}l{}{}".format(*s))
def test_scan_bwd_wide_dstate(shape):
    """d_state 33..128: every element of every gradient against the oracle
    (the slices' du, ddelta, dz summed, dA, dB, dC, dh0 placed per state,
    the skip term's dD from the first slice)."""
    b, d, n, L, io = shape
    x = I.scan_inputs(I.small_scan_config(b, d, n, L, io), with_h0=True)
    dy, dhl = grads_inputs(x)
    errs = check(run_gpu_bwd(x, dy, dhl), run_oracle_bwd(x, dy, dhl), io)
    print(shape, {k: f"{v:.1e}" for k, v in errs.items()})


@pytest.mark.parametrize("drop", [("D",), ("z",), ("D", "z")])
def test_scan_bwd_wide_optional_inputs(drop):
    x = I.scan_inputs(I.small_scan_config(2, 96, 64, 70, "fp32"))
    dy, _ = grads_inputs(x, with_dh_last=False)
    got = run_gpu_bwd(x, dy, None, drop=drop, with_h0=False)
    ref = run_oracle_bwd(x, dy, None, drop=drop, with_h0=False)
    if "D" in drop:
        ref_d = run_oracle_bwd(dict(x, D=np.zeros_like(x["D"])), dy, None, drop=tuple(k for k in drop if k != "D"),
                               with_h0=False)
        ref["dD"] = ref_d["dD"]
    check(got, ref, "fp32")


@pytest.mark.parametrize("force_general", [False, True])
def test_scan_bwd_wide_general_a(force_general):
    """A general in half the channels (per-state decay in every slice) and
    S4D-real in the rest (slices past the first see A[d, n0 + j], which the
    decay detection then treats as general)."""
    x = I.scan_inputs(I.small_scan_config(2, 128, 72, 90, "fp32"), with_h0=True)
    g = np.random.default_rng(5)
    x["A"] = (-np.exp(g.uniform(-1, 2, size=x["A"].shape))).astype(np.float32)
    x["A"][:64] = -(np.arange(72, dtype=np.float32) + 1)
    dy, dhl = grads_inputs(x)
    check(run_gpu_bwd(x, dy, dhl, force_general=force_general), run_oracle_bwd(x, dy, dhl), "fp32")


@pytest.mark.parametrize("shape", [(2, 12800, 64, 45, "bf16"), (1, 128, 48, 9000, "fp32")],
                         ids=["carry_handoff_n64", "split_passes_n48"])
def test_scan_bwd_wide_checkpoint_paths(shape):
    """The slices through the multi-workgroup paths: more streams than CUs
    (hand-offs) and few long sequences (split passes)."""
    b, d, n, L, io = shape
    x = I.scan_inputs(I.small_scan_config(b, d, n, L, io), with_h0=True)
    dy, dhl = grads_inputs(x)
    errs = check(run_gpu_bwd(x, dy, dhl), run_oracle_bwd(x, dy, dhl), io)
    print(shape, {k: f"{v:.1e}" for k, v in errs.items()})


def test_scan_bwd_wide_status_word():
    """The call's status word (first word of the workspace) is clear after a
    sliced backward with hand-offs between workgroups in every slice."""
    x = I.scan_inputs(I.small_scan_config(2, 12800, 40, 45, "bf16"), with_h0=True)
    dy, dhl = grads_inputs(x)
    g = {k: dev(x[k]) for k in ("u", "delta", "A", "B", "C", "D", "z", "h0")}
    ws = torch.full((mss.selective_scan_bwd_workspace_size(2, 12800, 40, 45, torch.bfloat16),), 255,
                    dtype=torch.uint8, device="cuda:0")
    mss.selective_scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], g["h0"], dy=dev(dy),
                           dh_last=dev(dhl), workspace=ws)
    assert mss.workspace_status(ws) == mss.MSS_OK


def test_scan_bwd_deterministic():
    x = I.scan_inputs(I.small_scan_config(2, 256, 16, 200, "bf16"), with_h0=True)
    dy, dhl = grads_inputs(x)
    a = run_gpu_bwd(x, dy, dhl)
    c = run_gpu_bwd(x, dy, dhl)
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], c[k]), k


def test_scan_bwd_2p8b_workload():
    """b=4, d_inner=5120, N=16, L=8192, bf16: the full backward launch; batch
    row 0 checked in full against the oracle (dB, dC of that row, du, ddelta,
    dz, dh0), dA and dD on sampled channels over all rows."""
    x = I.scan_inputs(I.SCAN_2P8B, with_h0=True)
    dy, dhl = grads_inputs(x)
    got = run_gpu_bwd(x, dy, dhl)
    ref = run_oracle_bwd(x, dy, dhl, rows=[0])
    row0 = {k: (None if v is None or k in ("dA", "dD") else v[:1]) for k, v in got.items()}
    errs = check(row0, ref, "bf16", keys=("du", "ddelta", "dB", "dC", "dz", "dh0"))
    chans = [0, 63, 64, 777, 2500, 5119]
    refc = run_oracle_bwd(x, dy, dhl, chans=chans)
    errs.update(check({"dA": got["dA"][chans], "dD": got["dD"][chans]}, refc, "bf16", keys=("dA", "dD")))
    print("scan_2p8b bwd:", {k: f"{v:.1e}" for k, v in errs.items()})
    assert rel_err(got["dh0"][:1], ref["dh0"]) < 1e-2


def test_scan_bwd_maximum_sizes_sampled():
    """At the documented limits (fp32, L = 2^24 - 5, dim*L just under 2^31,
    split passes): du, ddelta, dz, dA, dD of sampled channels against the
    oracle over the whole sequence (dB, dC sum over every channel and are
    left to the smaller cases).  Inputs drawn on the device (seeded)."""
    L = (1 << 24) - 5
    cfg = I.small_scan_config(1, 128, 16, L, "fp32", seed=I.SEED_BASE + 902)
    g = I.scan_inputs_device(cfg)
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(cfg.seed + 1)
    dy = torch.randn((1, 128, L), generator=gen, device="cuda:0", dtype=torch.float32)
    r = mss.selective_scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], dy=dy)
    torch.cuda.synchronize()
    chans = [0, 77, 127]
    h = lambda t: t.detach().cpu().numpy().astype(np.float64)
    ref = oracle.selective_scan_bwd(h(g["u"][:, chans]), h(g["delta"][:, chans]), h(g["A"][chans]), h(g["B"]),
                                    h(g["C"]), h(g["D"][chans]), h(g["z"][:, chans]), None, h(dy[:, chans]), None)
    errs = {}
    for k in ("du", "ddelta", "dz"):
        errs[k] = assert_close(h(r[k][:, chans]), ref[k], "fp32", k)
    for k in ("dA", "dD"):
        errs[k] = assert_close(h(r[k][chans]), ref[k], "fp32", k)
    print("bwd maximum sizes:", {k: f"{v:.1e}" for k, v in errs.items()})
