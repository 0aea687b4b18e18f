"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import numpy as np
import torch

from selective_state_space_27_amd import inputs as I

TOL = {"fp32": 1e-4, "bf16": 2e-2}


def dev(a, io=None):
    """numpy storage array -> contiguous torch tensor on cuda:0 (bf16 bits -> bfloat16)."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(a).to("cuda:0")


def host64(t):
    """torch tensor (fp32 or bf16, any device) -> fp64 numpy, exactly."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return I.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy().astype(np.float64)


def rel_err(got, ref):
    """max |g - r| / max(|r|, rms(r)) over the tensor (RMS floor for entries
    that cancel to near zero); NaN if shapes differ or non-finite values appear."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not np.all(np.isfinite(got)):
        return float("nan")
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    den = np.maximum(np.abs(ref), max(rms, 1e-300))
    return float(np.max(np.abs(got - ref) / den)) if ref.size else 0.0


def assert_close(got, ref, io, what=""):
    e = rel_err(got, ref)
    assert e <= TOL[io], f"{what}: max rel err {e:.3e} > {TOL[io]:.0e}"
    return e
