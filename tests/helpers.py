"""Shared helpers of the parity tests: tolerance rule and conversions."""
import numpy as np
import torch

# max |gpu - oracle| <= TOL * RMS(oracle), per compared tensor
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def f64(t) -> np.ndarray:
    """Exact widening of a (device or host) tensor to a float64 numpy array."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").to(torch.float64).numpy()


def rel_max_err(got, ref) -> float:
    got, ref = f64(got), f64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in the GPU result"
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


def assert_parity(got, ref, dtype, what: str):
    err = rel_max_err(got, ref)
    tol = TOL[dtype]
    print(f"[parity] {what}: max|err|/rms = {err:.3e} (tol {tol:.0e})", flush=True)
    assert err <= tol, f"{what}: max|err|/rms = {err:.3e} > {tol:.0e}"
    return err


def assert_parity_rounded(got, ref, tol: float, what: str, mant_bits: int = 8):
    """Parity of an output rounded once to a narrower float (bf16: 8 significant
    bits): elementwise |got - ref| <= tol*RMS(ref)*(1 + u) + u*|ref| with
    u = 2^-mant_bits the half-ulp bound of that final rounding, so the stated
    arithmetic tolerance is kept and only the output rounding is added."""
    g, r = f64(got), f64(ref)
    assert g.shape == r.shape and np.all(np.isfinite(g))
    u = 2.0 ** -mant_bits
    rms = float(np.sqrt(np.mean(r * r)))
    bound = tol * rms * (1 + u) + u * np.abs(r)
    excess = float(np.max(np.abs(g - r) - bound))
    worst = float(np.max(np.abs(g - r))) / max(rms, 1e-300)
    print(f"[parity] {what}: max|err|/rms = {worst:.3e}, tol {tol:.0e} + bf16 rounding, "
          f"margin {-excess / rms:.3e} rms", flush=True)
    assert excess <= 0, f"{what}: exceeds tol + rounding bound by {excess / rms:.3e} rms"
