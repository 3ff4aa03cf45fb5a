"""Helpers shared by the GPU parity tests: tolerances and device transfer."""
import json
import os

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


def log_margin(what, err, tol):
    """Append one parity margin to the JSON-lines file named by SSD_PARITY_LOG (if set)."""
    path = os.environ.get("SSD_PARITY_LOG")
    if path:
        case = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
        with open(path, "a") as fh:
            fh.write(json.dumps({"case": case, "what": what, "err": float(err), "tol": tol}) + "\n")


def check(out, ref, tol, what):
    e = rel_err(out, ref)
    print(f"  {what}: max|err|/max|ref| = {e:.3e} (bound {tol:.0e})", flush=True)
    log_margin(what, e, tol)
    assert e <= tol, f"{what}: relative error {e:.3e} exceeds {tol:.0e}"
    return e


def check_dev(out, ref, tol, what):
    """check() for two device tensors of any size, reduced on the device."""
    o, r = out.float(), ref.float()
    assert bool(torch.isfinite(o).all()), f"{what}: non-finite values"
    den = r.abs().max().item()
    e = (o - r).abs().max().item() / (den if den > 0 else 1.0)
    print(f"  {what}: max|diff|/max|ref| = {e:.3e} (bound {tol:.0e})", flush=True)
    log_margin(what, e, tol)
    assert e <= tol, f"{what}: relative difference {e:.3e} exceeds {tol:.0e}"
    return e
