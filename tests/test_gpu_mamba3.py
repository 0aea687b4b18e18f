"""GPU parity of mss_mamba3_state_update (one Mamba-3 generation step: the
trapezoid input rule, the complex rotating state and MIMO rank R, each an
option) against the fp64 oracle's step, through the C ABI.  Tolerance as for
the other calls: max |g - r| / max(|r|, rms(r)) <= 1e-4 for fp32 I/O and
2e-2 for bf16 I/O on y (bf16 outputs are rounded); the fp32 state meets
1e-4 in both."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_27_amd as mss
from selective_state_space_27_amd import inputs as I
from gpu_util import assert_close, dev, host64, rel_err

pytestmark = pytest.mark.gpu


def run_steps(cfg, steps, check_every=True, st=None):
    """`steps` consecutive steps on the GPU and in the oracle (x_prev/B_prev
    chained from the previous step when the trapezoid rule is on, zero before
    the first); compares y of every step (or the last) and the final state."""
    st = st or I.mamba3_static(cfg)
    h = dev(st["h0"])
    hr = st["h0"].astype(np.float64)
    A, D, th = dev(st["A"]), dev(st["D"]), dev(st["theta"])
    io = cfg.io
    zero_x = np.zeros((cfg.batch, cfg.nheads, cfg.rank, cfg.headdim), dtype=np.float64)
    zero_b = np.zeros((cfg.batch, cfg.ngroups, cfg.rank, cfg.dstate), dtype=np.float64)
    prev = None
    errs = []
    for s in range(steps):
        p = I.mamba3_step_inputs(cfg, s, st["dt"])
        g = {k: dev(p[k]) for k in ("x", "B", "C", "z", "delta")}
        if cfg.trapezoid:
            xp_d = g_prev["x"] if prev is not None else torch.zeros_like(g["x"])
            bp_d = g_prev["B"] if prev is not None else torch.zeros_like(g["B"])
        y = mss.mamba3_state_update(h, g["x"], g["delta"], A, g["B"], g["C"], D, g["z"],
                                    x_prev=xp_d if cfg.trapezoid else None, B_prev=bp_d if cfg.trapezoid else None,
                                    theta=th if cfg.complex_state else None)
        f = lambda k: I.to_f64(p[k], io)
        xp = (f64_prev["x"] if prev is not None else zero_x) if cfg.trapezoid else None
        bp = (f64_prev["B"] if prev is not None else zero_b) if cfg.trapezoid else None
        hr, yr = oracle.mamba3_step(hr, f("x"), p["delta"], st["A"], f("B"), f("C"), st["D"], f("z"), x_prev=xp,
                                    B_prev=bp, theta=st["theta"], complex_state=cfg.complex_state)
        if check_every or s == steps - 1:
            torch.cuda.synchronize()
            errs.append(assert_close(host64(y), yr, io, f"y step {s}"))
        prev, g_prev, f64_prev = p, g, {"x": f("x"), "B": f("B")}
    torch.cuda.synchronize()
    hg = host64(h)
    e_h = assert_close(hg, hr, "fp32", "state")
    return max(errs), e_h


CASES = [(c, t, r, io) for c in (False, True) for t in (False, True) for r in (1, 4) for io in ("fp32", "bf16")]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{'cplx' if c[0] else 'real'}-{'trap' if c[1] else 'euler'}-r{c[2]}-{c[3]}")
def test_mamba3_step_options(case):
    cplx, trap, R, io = case
    cfg = I.small_mamba3_config(3, 4, 32, 2, 128, R, 3, io, cplx, trap)
    ey, eh = run_steps(cfg, 3)
    print(f"{case}: y {ey:.2e} state {eh:.2e}")


@pytest.mark.parametrize("shape", [(2, 3, 16, 1, 64, 2), (1, 2, 128, 2, 256, 8), (2, 6, 64, 3, 64, 3)],
                         ids=lambda s: "b{}h{}p{}g{}n{}r{}".format(*s))
def test_mamba3_shapes(shape):
    b, H, P, G, N, R = shape
    cfg = I.small_mamba3_config(b, H, P, G, N, R, 2, "bf16", True, True)
    ey, eh = run_steps(cfg, 2)
    print(f"{shape}: y {ey:.2e} state {eh:.2e}")


def test_mamba3_many_steps_trapezoid_complex():
    """40 consecutive steps with the trapezoid input chained from step to step
    and the complex state: every step's outputs and the final state."""
    cfg = I.small_mamba3_config(2, 4, 32, 1, 128, 4, 40, "fp32", True, True, seed=I.SEED_BASE + 301)
    ey, eh = run_steps(cfg, 40)
    print(f"40 steps: y {ey:.2e} state {eh:.2e}")


def test_mamba3_rank1_real_euler_equals_state_update():
    """Rank 1, real state, Euler input is the Mamba-2 head's one-token update:
    the same step through mss_state_update, with channels (h, p), A[d, n] =
    A_h and delta[b, d] = delta[b, h], agrees."""
    cfg = I.small_mamba3_config(2, 3, 16, 1, 64, 1, 1, "fp32", False, False)
    st = I.mamba3_static(cfg)
    p = I.mamba3_step_inputs(cfg, 0, st["dt"])
    b, H, P, N = cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate
    h3 = dev(st["h0"])
    y3 = mss.mamba3_state_update(h3, dev(p["x"]), dev(p["delta"]), dev(st["A"]), dev(p["B"]), dev(p["C"]),
                                 dev(st["D"]), dev(p["z"]))
    h1 = dev(st["h0"].reshape(b, H * P, N))
    A1 = np.repeat(np.repeat(st["A"], P)[:, None], N, axis=1).astype(np.float32)
    y1 = mss.state_update(h1, dev(p["x"].reshape(b, H * P)), dev(np.repeat(p["delta"], P, axis=1)), dev(A1),
                          dev(p["B"].reshape(b, N)), dev(p["C"].reshape(b, N)), dev(np.repeat(st["D"], P)),
                          dev(p["z"].reshape(b, H * P)))
    torch.cuda.synchronize()
    assert rel_err(host64(y3).reshape(b, H * P), host64(y1)) < 1e-5
    assert rel_err(host64(h3).reshape(b, H * P, N), host64(h1)) < 1e-6


@pytest.mark.timeout(900)
def test_decode_m3_workload_full():
    """b=128, H=80, P=64, N=128, rank 4, complex state, trapezoid input, bf16
    I/O: three consecutive steps on the full state, every output element of
    each step and the whole state after the third against the oracle."""
    ey, eh = run_steps(I.DECODE_M3, 3)
    print(f"decode_m3 full, 3 steps: y max rel err {ey:.3e}, state {eh:.3e}")
