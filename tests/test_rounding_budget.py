"""Error budget of the bf16 path's rounding points, on the CPU.

The bf16 forward rounds at points the recurrence of the dbyun.net post (section "Mamba-2
架构") does not have, and at some where the post's kernels round differently (section
"Kernel 3：compute_out" keeps C B^T in fp32 up to its final product):

  xt    the state-pass operand x~ = bf16(wT x)                 (the post: bf16(dt decay B))
  S     chunk-start states stored in bf16                      (the post: cast to the input
                                                                type before its output product)
  corr  S_eff = bf16(S + beta bf16(H_g)) for grouped chains    (this design's grouping)
  cb    C B^T rounded to bf16 before the decay                 (the post: fp32)
  m     the decay matrix M' = CB exp(G_i - G_j) dt_j as a bf16 MFMA operand (the post: TF32)
  y     y rounded to bf16                                      (the post: the same)

Each point is emulated alone, in fp64 numpy, on the chunked algorithm with the GPU path's
grouping (chains split into groups of chunks, group-final states scanned, the carried state
added to each chunk-start state), and its error is measured against the fp64 oracle as
max|y - y_ref| / max|y_ref| (the GPU parity measure).  With no rounding point on, the
emulation equals the oracle to fp64 round-off, which pins it.  The bounds below are about
two to five times the measured figures; they document how the 2e-2 parity bound is
spent.  CPU only.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from state_space_sequence_cumsum_amd.inputs import Workload, make_inputs

POINTS = ("xt", "S", "corr", "cb", "m", "y")


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(torch.float64).numpy()


def emulate(inp, h, Q, K, on=()):
    """y [L, P] and hT [P, N] of head h (batch 0, one group) by the grouped chunked
    algorithm in fp64, with bf16 rounding at the points named in `on`."""
    r = (lambda a, p: bf16(a) if p in on else a)
    x = inp["x"][0, :, h, :].double().numpy()
    dt = inp["dt"][0, :, h].double().numpy()
    B = inp["B"][0, :, 0, :].double().numpy()
    C = inp["C"][0, :, 0, :].double().numpy()
    A = float(inp["A"][h])
    D = float(inp["D"][h])
    h0 = inp["h0"][0, h].double().numpy() if inp["h0"] is not None else None
    L, P = x.shape
    N = B.shape[1]
    nc = -(-L // Q)
    Lp = nc * Q
    pad = lambda a: np.concatenate([a, np.zeros((Lp - L,) + a.shape[1:])]) if Lp > L else a
    x, dt, B, C = pad(x), pad(dt), pad(B), pad(C)
    G = np.zeros(Lp)
    for c in range(nc):
        G[c * Q:(c + 1) * Q] = np.cumsum(A * dt[c * Q:(c + 1) * Q])
    glast = G[Q - 1::Q]
    ng = -(-nc // K)
    # grouped state pass: group g from zero (group 0 from h0), local chunk-start states
    S = np.zeros((nc, P, N))
    U = np.zeros((ng, P, N))
    beta = np.zeros(nc)
    gam = np.zeros(ng)
    for g in range(ng):
        st = h0.copy() if (g == 0 and h0 is not None) else np.zeros((P, N))
        run = 1.0
        for c in range(g * K, min((g + 1) * K, nc)):
            S[c] = r(st, "S")
            beta[c] = run
            sl = slice(c * Q, (c + 1) * Q)
            w = dt[sl] * np.exp(glast[c] - G[sl])
            xt = r(w[:, None] * x[sl], "xt")
            st = math.exp(glast[c]) * st + xt.T @ B[sl]
            run *= math.exp(glast[c])
        U[g] = st
        gam[g] = run
    # group scan: true group-start states
    Hg = np.zeros((ng, P, N))
    for g in range(1, ng):
        Hg[g] = gam[g - 1] * Hg[g - 1] + U[g - 1]
    hT = gam[ng - 1] * Hg[ng - 1] + U[ng - 1]
    # chunk output
    y = np.zeros((Lp, P))
    for c in range(nc):
        g = c // K
        S_eff = S[c] + beta[c] * r(Hg[g], "corr")
        S_eff = r(S_eff, "corr") if g > 0 else S_eff
        sl = slice(c * Q, (c + 1) * Q)
        Gc = G[sl]
        cb = r(C[sl] @ B[sl].T, "cb")
        i, j = np.meshgrid(np.arange(Q), np.arange(Q), indexing="ij")
        dec = np.where(i >= j, np.exp(np.minimum(Gc[:, None] - Gc[None, :], 0.0)), 0.0)
        M = r(cb * dec * dt[sl][None, :], "m")
        Y = np.exp(Gc)[:, None] * (C[sl] @ S_eff.T) + M @ x[sl]
        y[sl] = Y + D * x[sl]
    y = r(y[:L], "y")
    return y, hT


def _rel(a, ref):
    return float(np.abs(a - ref).max() / np.abs(ref).max())


# chunk 256, N = 256 as in the headline workload, 12 chunks in groups of 4; A scaled down for
# one head so that the carried group state matters (the headline's decay mostly hides it)
W = Workload("budget", "bf16", 1, 3072, 2, 64, 256, 1, 256, has_h0=True)
BOUND = {"xt": 4e-3, "S": 6e-3, "corr": 6e-3, "cb": 6e-3, "m": 6e-3, "y": 6e-3}


@pytest.fixture(scope="module")
def case():
    inp = make_inputs(W, 3)
    inp["A"][1] *= 1e-2
    ref = oracle.forward_full(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                              inp["h0"], chunk=W.chunk)
    return inp, ref


@pytest.mark.parametrize("h", [0, 1])
def test_emulation_without_rounding_is_the_oracle(case, h):
    inp, ref = case
    y, hT = emulate(inp, h, W.chunk, 4)
    assert _rel(y, ref["y"][0, :, h, :]) < 1e-10
    assert _rel(hT, ref["hT"][0, h]) < 1e-10


@pytest.mark.parametrize("h", [0, 1])
def test_each_rounding_point_within_its_budget(case, h):
    inp, ref = case
    yref = ref["y"][0, :, h, :]
    errs = {}
    for p in POINTS:
        y, _ = emulate(inp, h, W.chunk, 4, on=(p,))
        errs[p] = _rel(y, yref)
    y_all, _ = emulate(inp, h, W.chunk, 4, on=POINTS)
    errs["all"] = _rel(y_all, yref)
    print(f"  head {h}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for p in POINTS:
        assert errs[p] <= BOUND[p], (p, errs[p])
    assert errs["all"] <= 1e-2
