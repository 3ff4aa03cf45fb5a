"""Helpers shared by the GPU parity tests: tolerances and device transfer."""
import numpy as np
import torch

# max|out - ref| <= TOL * max|ref|, per tensor.  fp32 inputs: 1e-4; bf16 inputs with
# fp32 accumulation: 2e-2 (the required parity bar of the method).
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def require_gpu():
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return torch.device("cuda:0")


def to_dev(inp, dev):
    return {k: (None if v is None else v.to(dev)) for k, v in inp.items()}


def f64(t):
    return t.detach().float().cpu().double().numpy()


def rel_err(out, ref):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    assert np.isfinite(out).all(), "non-finite values in GPU output"
    den = np.abs(ref).max()
    return np.abs(out - ref).max() / (den if den > 0 else 1.0)


def check(out, ref, tol, what):
    e = rel_err(out, ref)
    print(f"  {what}: max|err|/max|ref| = {e:.3e} (bound {tol:.0e})", flush=True)
    assert e <= tol, f"{what}: relative error {e:.3e} exceeds {tol:.0e}"
    return e
