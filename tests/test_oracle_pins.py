"""Pins for the fp64 oracle, each against something other than the oracle itself.

Every check below comes from the mathematics of the recurrence on the
"Mamba-2 架构" section of dbyun.net's translation of the cuTile Mamba-2 post
(h_t = exp(A dt_t) h_{t-1} + dt_t x_t (outer) B_t, y_t = h_t . C_t + D x_t), its
unrolled and chunked rewrites (same page: the unrolled decayed sum, the log-space
jump h_next = exp(G_last) h + (exp(G_last - G) B)^T X, and the chunk output
Y = exp(G) C h + (exp(G_i - G_j) (C B^T) M) X + D X), the no-decay special case
(linear attention), or hand-worked values stored under tests/golden/.
The reference computations here are deliberately written differently from the
oracle (explicit products of exponentials, dense matrices, chunked algebra).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(seed, b=1, L=13, H=2, P=3, N=4, G=1, h0=True, dt_scale=0.7):
    rng = np.random.default_rng(seed)
    return {
        "x": rng.standard_normal((b, L, H, P)),
        "dt": np.abs(rng.standard_normal((b, L, H))) * dt_scale,
        "A": -np.exp(rng.uniform(0, math.log(4.0), H)),
        "B": rng.standard_normal((b, L, G, N)),
        "C": rng.standard_normal((b, L, G, N)),
        "D": rng.uniform(0, 1, H),
        "h0": rng.standard_normal((b, H, P, N)) if h0 else None,
    }


def _run(p, **kw):
    return oracle.forward_full(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"], **kw)


def _group(h, H, G):
    return h // (H // G)


# ---------------------------------------------------------------------------
# golden, hand-worked values
# ---------------------------------------------------------------------------
def test_golden_scalar():
    gd = json.load(open(os.path.join(GOLDEN, "scalar_L4.json")))
    L = len(gd["dt"])
    x = np.array(gd["x"]).reshape(1, L, 1, 1)
    dt = np.array(gd["dt"]).reshape(1, L, 1)
    B = np.array(gd["B"]).reshape(1, L, 1, 1)
    C = np.array(gd["C"]).reshape(1, L, 1, 1)
    for case in gd["cases"]:
        h0 = np.full((1, 1, 1, 1), case["h0"])
        out = oracle.forward_full(x, dt, gd["A"], B, C, gd["D"], h0, chunk=gd["chunk"])
        np.testing.assert_allclose(out["y"].ravel(), case["y"], rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(out["hT"].ravel(), [case["hT"]], rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(out["snaps"].ravel(), case["snaps"], rtol=1e-14, atol=1e-14)
    G2, dtc = oracle.chunk_cumsum(dt, gd["A"], gd["chunk"])
    np.testing.assert_allclose(G2.ravel(), gd["G2"], rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(dtc.ravel(), gd["dt"])


def test_golden_matrix_state_orientation():
    gd = json.load(open(os.path.join(GOLDEN, "p2_n3_L2.json")))
    x = np.array(gd["x"]).reshape(1, 2, 1, 2)
    dt = np.array(gd["dt"]).reshape(1, 2, 1)
    B = np.array(gd["B"]).reshape(1, 2, 1, 3)
    C = np.array(gd["C"]).reshape(1, 2, 1, 3)
    out = oracle.forward_full(x, dt, gd["A"], B, C, gd["D"], None)
    np.testing.assert_allclose(out["y"][0, :, 0, :], gd["y"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(out["hT"][0, 0], gd["hT"], rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------
# P1: brute-force unrolled sum with explicit products of exp(a_k)
# ---------------------------------------------------------------------------
def _brute_force(p):
    x, dt, A, B, C, D, h0 = (p[k] for k in ("x", "dt", "A", "B", "C", "D", "h0"))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.zeros((b, L, H, P))
    hT = np.zeros((b, H, P, N))
    for bi in range(b):
        for h in range(H):
            g = _group(h, H, G)
            e = [math.exp(A[h] * dt[bi, k, h]) for k in range(L)]

            def decay(lo, hi):  # product of exp(a_k) for k in [lo, hi]
                out = 1.0
                for k in range(lo, hi + 1):
                    out *= e[k]
                return out

            for t in range(L):
                for pp in range(P):
                    acc = 0.0
                    for j in range(t + 1):
                        cb = sum(C[bi, t, g, n] * B[bi, j, g, n] for n in range(N))
                        acc += decay(j + 1, t) * dt[bi, j, h] * cb * x[bi, j, h, pp]
                    if h0 is not None:
                        acc += decay(0, t) * sum(h0[bi, h, pp, n] * C[bi, t, g, n] for n in range(N))
                    y[bi, t, h, pp] = acc + D[h] * x[bi, t, h, pp]
            for pp in range(P):
                for n in range(N):
                    acc = decay(0, L - 1) * (h0[bi, h, pp, n] if h0 is not None else 0.0)
                    for j in range(L):
                        acc += decay(j + 1, L - 1) * dt[bi, j, h] * x[bi, j, h, pp] * B[bi, j, g, n]
                    hT[bi, h, pp, n] = acc
    return y, hT


@pytest.mark.parametrize("seed,shape", [(0, dict()), (1, dict(b=2, L=9, H=4, G=2, P=2, N=3)),
                                        (2, dict(L=1, h0=False)), (3, dict(L=17, H=3, G=3, P=2, N=5))])
def test_p1_brute_force_unrolled(seed, shape):
    p = _rand_problem(seed, **shape)
    y_bf, hT_bf = _brute_force(p)
    out = _run(p)
    scale = max(1.0, np.abs(y_bf).max())
    assert np.abs(out["y"] - y_bf).max() <= 1e-12 * scale
    assert np.abs(out["hT"] - hT_bf).max() <= 1e-12 * max(1.0, np.abs(hT_bf).max())


# ---------------------------------------------------------------------------
# P2: chunked (state-space-duality) algebra in numpy equals the sequential oracle
# ---------------------------------------------------------------------------
def _chunked(p, Q):
    x, dt, A, B, C, D, h0 = (p[k] for k in ("x", "dt", "A", "B", "C", "D", "h0"))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.zeros_like(x)
    hT = np.zeros((b, H, P, N))
    snaps = np.zeros((b, H, -(-L // Q), P, N))
    for bi in range(b):
        for h in range(H):
            g = _group(h, H, G)
            st = np.zeros((P, N)) if h0 is None else h0[bi, h].copy()
            for c, s in enumerate(range(0, L, Q)):
                e = min(L, s + Q)
                Xc, Bc, Cc, dtc = x[bi, s:e, h], B[bi, s:e, g], C[bi, s:e, g], dt[bi, s:e, h]
                Gc = np.cumsum(A[h] * dtc)                 # natural-log cumsum within the chunk
                snaps[bi, h, c] = st
                T = e - s
                causal = np.tril(np.ones((T, T), dtype=bool))
                with np.errstate(over="ignore"):
                    seg = np.where(causal, np.exp(Gc[:, None] - Gc[None, :]), 0.0)
                Yc = np.exp(Gc)[:, None] * (Cc @ st.T)
                Yc = Yc + (seg * (Cc @ Bc.T)) @ (dtc[:, None] * Xc)
                y[bi, s:e, h] = Yc + D[h] * Xc
                w = np.exp(Gc[-1] - Gc) * dtc
                st = math.exp(Gc[-1]) * st + (w[:, None] * Xc).T @ Bc
            hT[bi, h] = st
    return y, hT, snaps


@pytest.mark.parametrize("Q", [1, 2, 3, 7, 16, 64, 200])
def test_p2_chunked_equals_sequential(Q):
    p = _rand_problem(10 + Q, b=2, L=45, H=4, G=2, P=5, N=6, dt_scale=1.5)
    y_c, hT_c, snaps_c = _chunked(p, Q)
    out = _run(p, chunk=Q)
    assert np.abs(out["y"] - y_c).max() <= 1e-11 * np.abs(y_c).max()
    assert np.abs(out["hT"] - hT_c).max() <= 1e-11 * np.abs(hT_c).max()
    assert np.abs(out["snaps"] - snaps_c).max() <= 1e-11 * np.abs(snaps_c).max()


# ---------------------------------------------------------------------------
# P3: dt = 0 leaves the state unchanged (bitwise)
# ---------------------------------------------------------------------------
def test_p3_dt_zero_identity():
    p = _rand_problem(4, b=1, L=11, H=3, P=4, N=5)
    p["dt"][:] = 0.0
    out = _run(p)
    np.testing.assert_array_equal(out["hT"], p["h0"])
    ref = np.einsum("bhpn,blhn->blhp", p["h0"], p["C"][:, :, [0, 0, 0], :]) + p["D"][None, None, :, None] * p["x"]
    assert np.abs(out["y"] - ref).max() <= 1e-13 * np.abs(ref).max()


# ---------------------------------------------------------------------------
# P4: A = 0 turns the layer into causal linear attention (dense L x L matmul)
# ---------------------------------------------------------------------------
def test_p4_no_decay_is_causal_linear_attention():
    p = _rand_problem(5, b=2, L=23, H=2, G=1, P=3, N=4)
    p["A"][:] = 0.0
    out = _run(p)
    b, L, H, P = p["x"].shape
    mask = np.tril(np.ones((L, L)))
    for bi in range(b):
        for h in range(H):
            Cm, Bm = p["C"][bi, :, 0], p["B"][bi, :, 0]
            X = p["x"][bi, :, h]
            Y = Cm @ p["h0"][bi, h].T + ((Cm @ Bm.T) * mask) @ (p["dt"][bi, :, h][:, None] * X) + p["D"][h] * X
            assert np.abs(out["y"][bi, :, h] - Y).max() <= 1e-12 * np.abs(Y).max()
            hT = p["h0"][bi, h] + (p["dt"][bi, :, h][:, None] * X).T @ Bm
            assert np.abs(out["hT"][bi, h] - hT).max() <= 1e-12 * np.abs(hT).max()


# ---------------------------------------------------------------------------
# P5: continuation -- the final state is the next call's initial state
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("L1", [8, 5, 1])
def test_p5_continuation(L1):
    p = _rand_problem(6, b=1, L=16, H=2, P=3, N=4)
    full = _run(p)
    first = {k: (v[:, :L1] if k in ("x", "dt", "B", "C") else v) for k, v in p.items()}
    second = {k: (v[:, L1:] if k in ("x", "dt", "B", "C") else v) for k, v in p.items()}
    o1 = _run(first)
    second["h0"] = o1["hT"]
    o2 = _run(second)
    y = np.concatenate([o1["y"], o2["y"]], axis=1)
    assert np.abs(y - full["y"]).max() <= 1e-13 * np.abs(full["y"]).max()
    assert np.abs(o2["hT"] - full["hT"]).max() <= 1e-13 * np.abs(full["hT"]).max()


# ---------------------------------------------------------------------------
# P6: one token, closed form
# ---------------------------------------------------------------------------
def test_p6_single_token_closed_form():
    p = _rand_problem(7, b=1, L=1, H=2, P=3, N=4)
    out = _run(p)
    for h in range(2):
        a = p["A"][h] * p["dt"][0, 0, h]
        hT = math.exp(a) * p["h0"][0, h] + p["dt"][0, 0, h] * np.outer(p["x"][0, 0, h], p["B"][0, 0, 0])
        y = hT @ p["C"][0, 0, 0] + p["D"][h] * p["x"][0, 0, h]
        np.testing.assert_allclose(out["hT"][0, h], hT, rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(out["y"][0, 0, h], y, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# P7: linearity in (x, h0) jointly
# ---------------------------------------------------------------------------
def test_p7_linearity():
    p1 = _rand_problem(8, b=1, L=19, H=2, P=3, N=4)
    p2 = _rand_problem(9, b=1, L=19, H=2, P=3, N=4)
    p2.update({k: p1[k] for k in ("dt", "A", "B", "C", "D")})
    ps = dict(p1)
    ps["x"] = 2.0 * p1["x"] - 3.0 * p2["x"]
    ps["h0"] = 2.0 * p1["h0"] - 3.0 * p2["h0"]
    o1, o2, os_ = _run(p1), _run(p2), _run(ps)
    for k in ("y", "hT"):
        comb = 2.0 * o1[k] - 3.0 * o2[k]
        assert np.abs(os_[k] - comb).max() <= 1e-12 * np.abs(comb).max()


# ---------------------------------------------------------------------------
# P8: degenerate inputs
# ---------------------------------------------------------------------------
def test_p8_zero_C_and_zero_B():
    p = _rand_problem(11, b=1, L=10, H=2, P=3, N=4)
    pc = dict(p, C=np.zeros_like(p["C"]))
    out = _run(pc)
    np.testing.assert_allclose(out["y"], p["D"][None, None, :, None] * p["x"], rtol=0, atol=0)

    pb = dict(p, B=np.zeros_like(p["B"]))
    out = _run(pb)
    for h in range(2):
        run = 0.0
        for t in range(10):
            run += p["A"][h] * p["dt"][0, t, h]
            yt = math.exp(run) * (p["h0"][0, h] @ p["C"][0, t, 0]) + p["D"][h] * p["x"][0, t, h]
            np.testing.assert_allclose(out["y"][0, t, h], yt, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(out["hT"][0, h], math.exp(run) * p["h0"][0, h], rtol=1e-12, atol=0)


# ---------------------------------------------------------------------------
# P9: constant step, single impulse: geometric decay
# ---------------------------------------------------------------------------
def test_p9_geometric_impulse():
    p = _rand_problem(12, b=1, L=30, H=1, P=3, N=4, h0=False)
    p["dt"][:] = 0.37
    p["x"][:, 1:] = 0.0
    out = _run(p)
    a = p["A"][0] * 0.37
    base = 0.37 * np.outer(p["x"][0, 0, 0], p["B"][0, 0, 0])
    for t in range(30):
        ht = math.exp(a * t) * base
        np.testing.assert_allclose(out["y"][0, t, 0], ht @ p["C"][0, t, 0] + p["D"][0] * p["x"][0, t, 0],
                                   rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["hT"][0, 0], math.exp(a * 29) * base, rtol=1e-12, atol=0)


# ---------------------------------------------------------------------------
# head -> group mapping: heads use groups in contiguous blocks
# ---------------------------------------------------------------------------
def test_group_mapping_contiguous_blocks():
    p = _rand_problem(13, b=1, L=7, H=4, G=2, P=2, N=3, h0=False)
    p["B"][:, :, 1, :] = 0.0     # group 1 writes nothing into the state
    out = _run(p)
    Dx = p["D"][None, None, :, None] * p["x"]
    # heads 2 and 3 use group 1 -> pure skip connection; heads 0 and 1 do not
    np.testing.assert_array_equal(out["y"][:, :, 2:], Dx[:, :, 2:])
    assert np.abs(out["y"][:, :, :2] - Dx[:, :, :2]).max() > 1e-3


# ---------------------------------------------------------------------------
# cumsum pins (first kernel's output)
# ---------------------------------------------------------------------------
def test_cumsum_constant_step_closed_form():
    b, L, H, Q = 2, 50, 3, 16
    dt = np.full((b, L, H), 0.25)
    A = np.array([-1.0, -2.5, -16.0])
    G2, _ = oracle.chunk_cumsum(dt, A, Q)
    t = np.arange(L)
    for h in range(H):
        ref = math.log2(math.e) * A[h] * 0.25 * ((t % Q) + 1)
        np.testing.assert_allclose(G2[:, h], np.broadcast_to(ref, (b, L)), rtol=1e-13)


def test_cumsum_matches_recurrence_decay():
    """2^G2[t] is the decay the recurrence applies from the chunk start through token t."""
    rng = np.random.default_rng(14)
    L, Q = 40, 16
    dt = np.abs(rng.standard_normal((1, L, 1)))
    A = np.array([-0.8])
    G2, _ = oracle.chunk_cumsum(dt, A, Q)
    ones = np.ones((1, L, 1, 1))
    for t in range(L):
        s = (t // Q) * Q
        sub = lambda a: a[:, s:t + 1]
        o = oracle.forward_full(sub(ones), sub(dt), A, np.zeros((1, t + 1 - s, 1, 1)),
                                sub(ones), [0.0], np.ones((1, 1, 1, 1)))
        assert abs(2.0 ** G2[0, 0, t] - o["hT"].item()) <= 1e-13


# ---------------------------------------------------------------------------
# chunk-start snapshots are the states *before* each chunk
# ---------------------------------------------------------------------------
def test_snapshots_are_chunk_start_states():
    p = _rand_problem(15, b=1, L=21, H=2, P=3, N=4)
    Q = 5
    out = _run(p, chunk=Q)
    np.testing.assert_array_equal(out["snaps"][:, :, 0], p["h0"])
    for c in range(1, out["snaps"].shape[2]):
        pre = {k: (v[:, :c * Q] if k in ("x", "dt", "B", "C") else v) for k, v in p.items()}
        np.testing.assert_array_equal(out["snaps"][:, :, c], _run(pre)["hT"])


# ---------------------------------------------------------------------------
# storage types: bf16 inputs are widened exactly
# ---------------------------------------------------------------------------
def test_bf16_storage_widened_exactly():
    p = _rand_problem(16, b=1, L=12, H=2, P=3, N=4)
    tb = {k: torch.from_numpy(p[k]).to(torch.bfloat16) for k in ("x", "dt", "B", "C")}
    tf = {k: v.to(torch.float32) for k, v in tb.items()}
    o_b = oracle.forward_full(tb["x"], tb["dt"], p["A"], tb["B"], tb["C"], p["D"], p["h0"])
    o_f = oracle.forward_full(tf["x"], tf["dt"], p["A"], tf["B"], tf["C"], p["D"], p["h0"])
    np.testing.assert_array_equal(o_b["y"], o_f["y"])
    np.testing.assert_array_equal(o_b["hT"], o_f["hT"])
    G_b, d_b = oracle.chunk_cumsum(tb["dt"], p["A"], 4)
    np.testing.assert_array_equal(d_b.transpose(0, 2, 1), tf["dt"].double().numpy())


def test_unit_subset_and_thread_count_invariance():
    p = _rand_problem(17, b=2, L=15, H=3, G=3, P=2, N=3)
    full = oracle.forward(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"], nthreads=1)
    sub = oracle.forward(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"],
                         units=[5, 1, 3], nthreads=3)
    for i, u in enumerate([5, 1, 3]):
        np.testing.assert_array_equal(sub["y"][i], full["y"][u])
        np.testing.assert_array_equal(sub["hT"][i], full["hT"][u])


def test_bad_arguments_rejected():
    p = _rand_problem(18, b=1, L=4, H=3, G=1, P=2, N=2)
    with pytest.raises(ValueError):
        oracle.forward(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], units=[99])
    with pytest.raises(ValueError):
        oracle.forward(p["x"], p["dt"], p["A"][:2], p["B"], p["C"], p["D"])
    bad = dict(p, B=np.zeros((1, 4, 2, 2)), C=np.zeros((1, 4, 2, 2)))   # H=3 not divisible by G=2
    with pytest.raises(ValueError):
        _run(bad)
