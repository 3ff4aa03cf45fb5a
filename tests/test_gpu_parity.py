"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every case draws seeded inputs from the shared recipe, runs libssd on cuda:0
and compares element by element with the oracle run on the very same stored
values.  Per tensor the bar is max|out - ref| <= tau * max|ref| with tau = 1e-4
for fp32 inputs and 2e-2 for bf16 inputs (fp32 accumulation).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import state_space_sequence_cumsum_amd as ssd
from state_space_sequence_cumsum_amd.inputs import WORKLOADS, Workload, make_inputs
from gpu_util import TOL, check, check_dev, f64, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _wl(name="t", dtype="bf16", b=1, L=256, H=4, P=64, N=64, G=1, Q=64, h0=True, shift=-4.0):
    return Workload(name, dtype, b, L, H, P, N, G, Q, dt_shift=shift, has_h0=h0)


def _gpu_forward(inp, w, dev, poison=True):
    d = to_dev(inp, dev)
    io = d["x"].dtype
    y = torch.empty(w.batch, w.seqlen, w.nheads, w.headdim, device=dev, dtype=io)
    hT = torch.empty(w.batch, w.nheads, w.headdim, w.dstate, device=dev, dtype=torch.float32)
    if poison:
        y.fill_(float("nan"))
        hT.fill_(float("nan"))
    prob = ssd.problem_of(d["x"], d["B"], w.chunk)
    ws = ssd.workspace_for(prob, dev)
    ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk,
                    y=y, hT=hT, workspace=ws)
    torch.cuda.synchronize()
    return y, hT, ws, prob


def _stage_states(inp, w, dev):
    """True chunk-start states and final state from the public stage-1 and stage-2
    entry points (one serial chain per (batch, head) and N tile)."""
    d = to_dev(inp, dev)
    prob = ssd.problem_of(d["x"], d["B"], w.chunk)
    G2, dtT = ssd.ssd_chunk_cumsum(prob, d["dt"], d["A"])
    S = torch.full((w.batch, w.nheads, w.nchunks, w.headdim, w.dstate), float("nan"),
                   device=dev, dtype=d["x"].dtype)
    S, hT = ssd.ssd_state_pass(prob, d["x"], d["B"], G2, dtT, d["h0"], S=S)
    torch.cuda.synchronize()
    return S, hT


def _check_forward(w, seed=0, inp=None, dev=None):
    dev = dev or require_gpu()
    inp = inp or make_inputs(w, seed)
    print(f"case {w} seed={seed}", flush=True)
    y, hT, ws, prob = _gpu_forward(inp, w, dev)
    ref = oracle.forward_full(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                              inp["h0"], chunk=w.chunk)
    tol = TOL[w.dtype]
    check(f64(y), ref["y"], tol, "y")
    check(f64(hT), ref["hT"], tol, "hT")
    S, hT2 = _stage_states(inp, w, dev)
    check(f64(S), ref["snaps"], tol, "chunk-start states (stage 2)")
    check(f64(hT2), ref["hT"], tol, "hT (stage 2)")
    return y, hT, ref


# ---------------------------------------------------------------------------
# stage 1 alone
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,L,H,Q", [("fp32", 256, 4, 64), ("bf16", 2048, 24, 256),
                                         ("bf16", 200, 33, 64), ("bf16", 1000, 7, 128)])
def test_chunk_cumsum_parity(dtype, L, H, Q):
    dev = require_gpu()
    w = _wl(dtype=dtype, b=2, L=L, H=H, Q=Q)
    inp = make_inputs(w, 3)
    prob = ssd.problem_of(inp["x"], inp["B"], Q)
    G2, dtT = ssd.ssd_chunk_cumsum(prob, inp["dt"].to(dev), inp["A"].to(dev))
    torch.cuda.synchronize()
    G2_ref, dt_ref = oracle.chunk_cumsum(inp["dt"], inp["A"], Q)
    G2g, dtg = f64(G2), f64(dtT)
    # valid tokens: G2 within the fp32 summation bound, dtT exactly fp32(dt)
    bound = (Q + 2) * 2.0 ** -24 * max(1.0, np.abs(G2_ref).max())
    err = np.abs(G2g[:, :, :L] - G2_ref).max()
    print(f"  G2 max|err| = {err:.3e} (bound {bound:.3e})")
    assert err <= bound
    np.testing.assert_array_equal(dtg[:, :, :L], dt_ref)
    # padded tail: dt = 0 and the cumsum frozen at the last valid token (the state pass
    # reads the chunk's decay at its last position)
    if G2g.shape[2] > L:
        assert (dtg[:, :, L:] == 0).all()
        np.testing.assert_array_equal(G2g[:, :, L:], np.repeat(G2g[:, :, L - 1:L], G2g.shape[2] - L, 2))


# ---------------------------------------------------------------------------
# whole forward, small shapes spanning tiles, ragged tails and every template
# ---------------------------------------------------------------------------
SMALL_CASES = [
    _wl("fp32_small", "fp32", 1, 256, 4, 64, 64, 1, 64, h0=False),   # the small fp32 workload
    _wl("fp32_tail", "fp32", 2, 200, 3, 64, 128, 1, 64),
    _wl("fp32_q128", "fp32", 1, 384, 2, 64, 64, 2, 128),
    _wl("fp32_q256", "fp32", 1, 300, 2, 64, 64, 1, 256),
    _wl("bf16_q64_n64", "bf16", 2, 512, 4, 64, 64, 2, 64),
    _wl("bf16_q128_n128", "bf16", 1, 640, 4, 64, 128, 1, 128),
    _wl("bf16_q256_n256", "bf16", 1, 1024, 3, 64, 256, 3, 256),
    _wl("bf16_q128_n512", "bf16", 1, 384, 2, 64, 512, 1, 128),
    _wl("bf16_tail_q256", "bf16", 2, 700, 2, 64, 192, 1, 256),
    _wl("bf16_short", "bf16", 1, 37, 2, 64, 64, 1, 128),
    _wl("bf16_one_token", "bf16", 1, 1, 2, 64, 64, 1, 64),
    # many state-pass groups, ragged last chunk, groups of uneven length
    _wl("bf16_groups_q128", "bf16", 1, 3000, 2, 64, 128, 1, 128),
    _wl("bf16_groups_q256", "bf16", 2, 2900, 3, 64, 256, 3, 256),
    _wl("bf16_groups_q64", "bf16", 1, 1100, 1, 64, 64, 1, 64, h0=False),
    _wl("bf16_groups_q64_n256", "bf16", 1, 1500, 2, 64, 256, 1, 64),   # S_eff staged in 2 rounds
    _wl("bf16_groups_odd", "bf16", 1, 1100, 43, 64, 256, 1, 128),   # 3 chunks per group
    # N = 512 with 128-token chunks: column halves split over wave pairs
    _wl("bf16_groups_n512", "bf16", 1, 2200, 4, 64, 512, 2, 128),    # grouped, ragged, G = 2
    _wl("bf16_hb2_n512", "bf16", 1, 8192, 8, 64, 512, 1, 128),       # 2 heads per block
    # corners of the supported set on the single-head chunk output
    _wl("bf16_q64_n512", "bf16", 1, 300, 2, 64, 512, 1, 64),
    # the register-transposed state pass (N = 512): one sub-step per chunk over many groups,
    # and a sequence shorter than one sub-step
    _wl("bf16_rt_q64_groups", "bf16", 1, 2050, 2, 64, 512, 1, 64),
    _wl("bf16_rt_short", "bf16", 2, 45, 2, 64, 512, 2, 256),
    _wl("bf16_q256_n512", "bf16", 1, 600, 2, 64, 512, 2, 256, shift=-3.0),
    _wl("bf16_q128_n448", "bf16", 2, 500, 3, 64, 448, 1, 128),
    _wl("bf16_q256_n384", "bf16", 1, 700, 4, 64, 384, 4, 256, h0=False),
    _wl("fp32_q128_n512", "fp32", 1, 260, 2, 64, 512, 1, 128),
    # fp32 state pass split into groups: one chunk per group with a ragged last chunk,
    # and two chunks per group with G = 2 and h0
    _wl("fp32_groups_k1", "fp32", 1, 3000, 2, 64, 128, 1, 128, h0=False),
    _wl("fp32_groups_k2", "fp32", 2, 2000, 8, 64, 256, 2, 256),
]


@pytest.mark.parametrize("w", SMALL_CASES, ids=[c.name for c in SMALL_CASES])
def test_forward_parity_small(w):
    _check_forward(w, seed=0)


# many heads over short sequences: the state pass runs as one group per (batch, head), and the
# chunk output reads true chunk-start states (its uncorrected instances)
SINGLE_GROUP_CASES = [
    _wl("sg_hb_n64_q128", "bf16", 2, 320, 128, 64, 64, 1, 128),            # 4 heads per block, ragged
    _wl("sg_hb_n256_q256", "bf16", 1, 640, 128, 64, 256, 1, 256, h0=False),
    _wl("sg_hb_n256_q128", "bf16", 1, 320, 96, 64, 256, 2, 128),
    _wl("sg_hb_n512_q128", "bf16", 1, 256, 256, 64, 512, 1, 128),         # column halves
    _wl("sg_onehead_q64", "bf16", 1, 160, 96, 64, 128, 3, 64),
    _wl("sg_fp32_q256", "fp32", 1, 640, 64, 64, 256, 1, 256),
    _wl("sg_fp32_q128", "fp32", 1, 320, 128, 64, 256, 2, 128, h0=False),
    _wl("sg_fp32_q64", "fp32", 4, 160, 128, 64, 128, 1, 64),
]


@pytest.mark.parametrize("w", SINGLE_GROUP_CASES, ids=[c.name for c in SINGLE_GROUP_CASES])
def test_forward_parity_single_group(w):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    prob = ssd.make_problem(w.batch, w.seqlen, w.nheads, w.ngroups, w.headdim, w.dstate, w.chunk, dt)
    assert ssd.ssd_plan(prob)["sp_groups"] == 1, "shape no longer runs as one group"
    _check_forward(w, seed=3)


def _random_cases(n, seed=2026):
    """n shapes drawn from the supported set (any L, H divisible by G, N a multiple of 64 up
    to 512, Q in {64, 128, 256}, bf16 or fp32, with or without h0), sized for the oracle."""
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        Q = int(rng.choice([64, 128, 256]))
        N = int(64 * rng.integers(1, 9))
        G = int(rng.choice([1, 2, 3]))
        H = G * int(rng.integers(1, 4))
        b = int(rng.integers(1, 3))
        L = int(rng.integers(1, 1500))
        dtype = "fp32" if rng.random() < 0.25 else "bf16"
        cases.append(_wl(f"rand{k}_{dtype}_b{b}L{L}H{H}G{G}N{N}Q{Q}", dtype, b, L, H, 64, N, G, Q,
                         h0=bool(rng.random() < 0.6), shift=float(rng.choice([-4.0, -2.0, 0.0]))))
    return cases


RANDOM_CASES = _random_cases(12)


@pytest.mark.parametrize("w", RANDOM_CASES, ids=[c.name for c in RANDOM_CASES])
def test_forward_parity_random_shapes(w):
    _check_forward(w, seed=7)


@pytest.mark.parametrize("seed", [1, 2])
def test_forward_parity_seeds(seed):
    _check_forward(_wl("bf16_seeds", "bf16", 1, 512, 4, 64, 128, 1, 128), seed=seed)


# ---------------------------------------------------------------------------
# special cases and adversarial numerics
# ---------------------------------------------------------------------------
def test_dt_zero_keeps_state_bitwise():
    dev = require_gpu()
    w = _wl("dt0", "bf16", 1, 300, 2, 64, 128, 1, 128)
    inp = make_inputs(w, 4)
    inp["dt"].zero_()
    y, hT, _, _ = _gpu_forward(inp, w, dev)
    torch.testing.assert_close(hT.cpu(), inp["h0"], rtol=0, atol=0)
    ref = oracle.forward_full(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"])
    check(f64(y), ref["y"], TOL["bf16"], "y (dt = 0)")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_no_decay_linear_attention(dtype):
    w = _wl("A0", dtype, 1, 320, 2, 64, 64, 1, 64)
    inp = make_inputs(w, 5)
    inp["A"].zero_()
    _check_forward(w, inp=inp)


WEAK_DECAY = [
    _wl("weak_decay_n128", "bf16", 1, 4096, 4, 64, 128, 1, 128),
    _wl("weak_decay_n256", "bf16", 2, 3000, 3, 64, 256, 1, 256),
    _wl("weak_decay_n512", "bf16", 1, 3000, 2, 64, 512, 2, 128),     # register-transposed state pass
    _wl("weak_decay_fp32", "fp32", 1, 3000, 2, 64, 128, 1, 128),
]


@pytest.mark.parametrize("w", WEAK_DECAY, ids=[c.name for c in WEAK_DECAY])
def test_grouped_weak_decay(w):
    """A scaled by 1e-3: the decay over the whole sequence stays above one half, so the
    state a group of chunks inherits (the group scan's carried state and the S + beta H
    correction of the chunk output) is most of every chunk-start state and of hT."""
    dev = require_gpu()
    inp = make_inputs(w, 12)
    inp["A"].mul_(1e-3)
    total = (inp["A"][None, :] * inp["dt"].float().sum(dim=1)).exp()
    assert float(total.min()) > 0.5
    assert ssd.ssd_plan(ssd.problem_of(inp["x"], inp["B"], w.chunk))["sp_groups"] > 1
    _check_forward(w, inp=inp, dev=dev)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_masked_exponent_overflow(dtype):
    """A = -16 and dt near 1: within a chunk |G2| passes 128, so the masked upper
    triangle holds exp2 of large positive numbers (+inf); selection must drop them."""
    w = _wl("overflow", dtype, 1, 512, 2, 64, 64, 1, 256)
    inp = make_inputs(w, 6)
    inp["A"].fill_(-16.0)
    inp["dt"] = (0.9 + 0.2 * torch.rand(inp["dt"].shape, generator=torch.Generator().manual_seed(6))).to(inp["dt"].dtype)
    G2_ref, _ = oracle.chunk_cumsum(inp["dt"], inp["A"], w.chunk)
    assert np.abs(G2_ref).max() > 1000
    _check_forward(w, inp=inp)


def test_masked_exponent_overflow_one_launch():
    """The same on the one-launch fp32 forward (64-token chunks, dstate 64, 8 chunks): within
    a chunk |G2| passes 1000, and its C B^T tiles select on i >= j as well."""
    w = _wl("overflow_one_launch", "fp32", 1, 480, 2, 64, 64, 1, 64)
    inp = make_inputs(w, 6)
    inp["A"].fill_(-16.0)
    inp["dt"] = 0.9 + 0.2 * torch.rand(inp["dt"].shape, generator=torch.Generator().manual_seed(6))
    assert ssd.ssd_plan(ssd.problem_of(inp["x"], inp["B"], w.chunk))["fused"] == 1
    G2_ref, _ = oracle.chunk_cumsum(inp["dt"], inp["A"], w.chunk)
    assert np.abs(G2_ref).max() > 1000
    _check_forward(w, inp=inp)


@pytest.mark.parametrize("zero", ["B", "C"])
def test_degenerate_zero_B_or_C_one_launch(zero):
    """B = 0 or C = 0 on the one-launch fp32 forward (ragged, 5 chunks): with C = 0, y equals
    D x rounded once, bit for bit."""
    w = _wl(f"zero_{zero}_one_launch", "fp32", 2, 300, 3, 64, 64, 1, 64)
    inp = make_inputs(w, 8)
    inp[zero].zero_()
    if zero == "B":
        inp["A"].mul_(0.01)
    assert ssd.ssd_plan(ssd.problem_of(inp["x"], inp["B"], w.chunk))["fused"] == 1
    y, hT, ref = _check_forward(w, inp=inp)
    if zero == "C":
        skip = inp["D"][None, None, :, None] * inp["x"]
        assert torch.equal(y.cpu(), skip)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("zero", ["B", "C"])
def test_degenerate_zero_B_or_C(dtype, zero):
    """B = 0: nothing enters the state, so hT = exp(sum of a) h0 and y_t = exp(G_t) C_t h0
    + D x_t (the grouped state pass then carries only h0 through the group scan).  C = 0:
    the state is never read out and y = D x; the chunk output rounds the fp32 product once,
    so y equals round(D x) bit for bit.  With B = 0, A is scaled by 0.01 so that h0 is
    still well above fp32's range at the end (with A down to -16 the exact hT is ~1e-50)."""
    Q = 128 if dtype == "bf16" else 64
    w = _wl(f"zero_{zero}", dtype, 1, 700, 3, 64, 128, 1, Q)
    inp = make_inputs(w, 8)
    inp[zero].zero_()
    if zero == "B":
        inp["A"].mul_(0.01)
    y, hT, ref = _check_forward(w, inp=inp)
    if zero == "C":
        skip = (inp["D"][None, None, :, None] * inp["x"].float()).to(inp["x"].dtype)
        assert torch.equal(y.cpu(), skip)


def test_state_continuation():
    dev = require_gpu()
    w = _wl("cont", "fp32", 1, 448, 2, 64, 64, 1, 64)
    inp = make_inputs(w, 7)
    y_full, hT_full, _, _ = _gpu_forward(inp, w, dev)
    for L1 in (192, 100):   # chunk-aligned and unaligned split
        a = {k: (v[:, :L1].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
        bb = {k: (v[:, L1:].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
        y1, hT1, _, _ = _gpu_forward(a, w.with_(seqlen=L1), dev)
        bb["h0"] = hT1.cpu()
        y2, hT2, _, _ = _gpu_forward(bb, w.with_(seqlen=w.seqlen - L1), dev)
        check(f64(torch.cat([y1, y2], 1)), f64(y_full), TOL["fp32"], f"y split at {L1}")
        check(f64(hT2), f64(hT_full), TOL["fp32"], f"hT split at {L1}")


def test_h0_and_hT_may_alias():
    dev = require_gpu()
    w = _wl("alias", "bf16", 1, 256, 2, 64, 128, 1, 128)
    inp = make_inputs(w, 8)
    d = to_dev(inp, dev)
    ref = oracle.forward_full(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"])
    state = d["h0"].clone()
    y, hT = ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], state, chunk=w.chunk,
                            hT=state)
    torch.cuda.synchronize()
    check(f64(state), ref["hT"], TOL["bf16"], "hT written over h0")
    check(f64(y), ref["y"], TOL["bf16"], "y")


def test_deterministic_bitwise():
    dev = require_gpu()
    w = _wl("det", "bf16", 1, 1024, 4, 64, 256, 1, 256)
    inp = make_inputs(w, 9)
    y1, h1, _, _ = _gpu_forward(inp, w, dev)
    y2, h2, _, _ = _gpu_forward(inp, w, dev)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_stages_match_forward(dtype):
    """The public stages (one serial chain) and ssd_forward (grouped state pass with the
    carried state added in stage 3) agree with each other and with the oracle."""
    dev = require_gpu()
    w = _wl("stages", dtype, 2, 1280, 4, 64, 128, 2, 64)
    inp = make_inputs(w, 10)
    d = to_dev(inp, dev)
    prob = ssd.problem_of(d["x"], d["B"], w.chunk)
    G2, dtT = ssd.ssd_chunk_cumsum(prob, d["dt"], d["A"])
    S, hT = ssd.ssd_state_pass(prob, d["x"], d["B"], G2, dtT, d["h0"])
    y = ssd.ssd_chunk_out(prob, d["x"], d["B"], d["C"], G2, dtT, S, d["D"])
    yf, hTf, _, _ = _gpu_forward(inp, w, dev)
    ref = oracle.forward_full(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"])
    assert ssd.ssd_plan(prob)["sp_groups"] > 1
    check(f64(y), ref["y"], TOL[dtype], "y (stages)")
    check(f64(yf), ref["y"], TOL[dtype], "y (forward)")
    check(f64(hTf), f64(hT), 1e-5, "hT forward vs stages (both fp32 states)")


STAGE1_CASES = [
    _wl("s1_groups_q128", "bf16", 1, 3000, 2, 64, 128, 1, 128),     # grouped, ragged
    _wl("s1_n512_q128", "bf16", 1, 1000, 2, 64, 512, 2, 128),       # two state-pass column workgroups
    _wl("s1_q64", "bf16", 2, 650, 3, 64, 64, 1, 64),
    _wl("s1_q256", "bf16", 1, 2900, 3, 64, 256, 3, 256, shift=-2.0),
    _wl("s1_fp32", "fp32", 1, 300, 2, 64, 64, 1, 64),
]


@pytest.mark.parametrize("w", STAGE1_CASES, ids=[c.name for c in STAGE1_CASES])
def test_forward_stage1_outputs_match_stage1_bitwise(w):
    """What ssd_forward leaves in its workspace as stage-1 output (G2, dtT) equals the
    stage-1 entry point's output bit for bit, on every element."""
    dev = require_gpu()
    inp = make_inputs(w, 21)
    print(f"case {w}", flush=True)
    d = to_dev(inp, dev)
    prob = ssd.problem_of(d["x"], d["B"], w.chunk)
    ws = ssd.workspace_for(prob, dev)
    ws.fill_(0xFF)   # NaN patterns: every element must be written
    ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk,
                    workspace=ws)
    G2, dtT = ssd.ssd_chunk_cumsum(prob, d["dt"], d["A"])
    torch.cuda.synchronize()
    v = ssd.workspace_views(prob, ws)
    for name, ref in (("G2", G2), ("dtT", dtT)):
        assert torch.equal(v[name], ref), name


@pytest.mark.parametrize("w", [_wl("nofinal_groups", "bf16", 1, 3000, 2, 64, 128, 1, 128),
                               _wl("nofinal_fp32", "fp32", 1, 300, 2, 64, 64, 1, 64)],
                         ids=["bf16-grouped", "fp32"])
def test_forward_without_final_state(w):
    """hT = NULL (want_final=False): the same y, bit for bit, and nothing else written."""
    dev = require_gpu()
    inp = make_inputs(w, 31)
    d = to_dev(inp, dev)
    y1, h1 = ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk)
    y2, h2 = ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk,
                             want_final=False)
    torch.cuda.synchronize()
    assert h2 is None and torch.equal(y1, y2)


def test_forward_timed_events():
    dev = require_gpu()
    w = _wl("timed", "bf16", 1, 1024, 2, 64, 128, 1, 128)
    inp = make_inputs(w, 12)
    d = to_dev(inp, dev)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(ssd.FORWARD_EVENTS)]
    for e in evs:
        e.record()
    y1, h1 = ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk,
                             events=evs)
    y2, h2 = ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    times = [evs[i].elapsed_time(evs[i + 1]) for i in range(ssd.FORWARD_EVENTS - 1)]
    assert all(t >= 0 for t in times), times
    with pytest.raises(ValueError):
        ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk,
                        events=evs[:4])


@pytest.mark.parametrize("w", [_wl("stages_grouped", "bf16", 1, 4096, 4, 64, 128, 1, 256),
                               _wl("stages_ragged", "bf16", 2, 1000, 4, 64, 64, 2, 128),
                               _wl("stages_fp32", "fp32", 1, 1024, 2, 64, 64, 1, 64)],
                         ids=lambda w: w.name)
def test_forward_stages_one_at_a_time(w):
    """ssd_forward_stage 0, 1, 2, 3 in order reproduces ssd_forward bit for bit; repeating
    stage 3 (and stage 0) on the filled workspace recomputes the same outputs."""
    dev = require_gpu()
    d = to_dev(make_inputs(w, 4), dev)
    y_ref, h_ref = ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                                   chunk=w.chunk)
    plan = ssd.ForwardPlan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk)
    plan.y.fill_(float("nan"))
    plan.hT.fill_(float("nan"))
    for stage in range(4):
        plan.run_stage(stage)
    torch.cuda.synchronize()
    assert torch.equal(plan.y, y_ref) and torch.equal(plan.hT, h_ref)
    plan.y.fill_(float("nan"))
    for stage in (3, 0, 3):
        plan.run_stage(stage)
    torch.cuda.synchronize()
    assert torch.equal(plan.y, y_ref)


def test_errors_before_launch():
    dev = require_gpu()
    w = _wl("err", "bf16", 1, 128, 2, 64, 64, 1, 64)
    d = to_dev(make_inputs(w, 11), dev)
    with pytest.raises(ValueError):
        ssd.ssd_forward(d["x"].cpu(), d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=64)
    with pytest.raises(ssd.SsdError) as ei:
        ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=96)
    assert ei.value.status == 3
    prob = ssd.problem_of(d["x"], d["B"], 64)
    small = torch.empty(16, device=dev, dtype=torch.uint8)
    with pytest.raises(ssd.SsdError) as ei:
        ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=64, workspace=small)
    assert ei.value.status == 4


# ---------------------------------------------------------------------------
# the study workloads and the pages' example at full size, in the benchmark's launch configuration;
# the oracle computes a sample of (batch, head) units over the whole sequence
# ---------------------------------------------------------------------------
FULL = [(name, units) for name, units in [
    ("fp32_b1_L256_H4_P64_N64_Q64", None),
    ("bf16_b2_L2048_H24_P64_N128_Q256", [0, 13, 23, 24, 40, 47]),
    ("bf16_b1_L16384_H32_P64_N256_Q256", [0, 17, 31]),
    ("bf16_b1_L65536_H32_P64_N512_Q128", [5, 30]),
    ("bf16_b1_L262144_H16_G2_P64_N128_Q256", [2, 12]),
    ("bf16_b4_L16384_H8_P64_N128_Q128", [0, 11, 31]),
]]


@pytest.mark.slow
@pytest.mark.parametrize("name,units", FULL, ids=[n for n, _ in FULL])
def test_full_workload_sampled(name, units):
    dev = require_gpu()
    w = WORKLOADS[name]
    inp = make_inputs(w, 0)
    print(f"case {name}: units {units}", flush=True)
    y, hT, ws, prob = _gpu_forward(inp, w, dev)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"],
                         units=units, chunk=w.chunk)
    u = ref["units"]
    b_idx, h_idx = u // w.nheads, u % w.nheads
    y_s = np.stack([f64(y[b, :, h, :]) for b, h in zip(b_idx, h_idx)])
    tol = TOL[w.dtype]
    check(y_s, ref["y"], tol, "y (sampled units)")
    check(np.stack([f64(hT[b, h]) for b, h in zip(b_idx, h_idx)]), ref["hT"], tol, "hT (sampled units)")
    # every (batch, head) of the forward (grouped state pass, group scan, head-blocked
    # chunk output) against the plain stage path (one serial state chain per head, the
    # ungrouped chunk output), which runs other kernel instances: both sides are within
    # the bound of the oracle, so their difference is bounded by it too
    d = to_dev(inp, dev)
    G2, dtT = ssd.ssd_chunk_cumsum(prob, d["dt"], d["A"])
    S, hT2 = ssd.ssd_state_pass(prob, d["x"], d["B"], G2, dtT, d["h0"])
    check(np.stack([f64(S[b, h]) for b, h in zip(b_idx, h_idx)]), ref["snaps"], tol,
          "chunk-start states (stage 2, sampled units)")
    y2 = ssd.ssd_chunk_out(prob, d["x"], d["B"], d["C"], G2, dtT, S, d["D"])
    torch.cuda.synchronize()
    check_dev(y, y2, tol, "y, every unit: forward against the stage path")
    check_dev(hT, hT2, tol, "hT, every unit: forward against the stage path")
    del S, y2, G2, dtT


@pytest.mark.slow
def test_largest_batch_heads_sampled():
    """batch * heads at the supported maximum (65535, a grid dimension of the group scan and
    of the one-head chunk output): 4369 sequences of 15 heads in 3 groups, 200 tokens in
    128-token chunks (one full, one ragged), so the state pass runs as one group and both
    chunk-output kernels run their largest grids; sampled units against the oracle."""
    dev = require_gpu()
    w = _wl("max_bh", "bf16", 4369, 200, 15, 64, 64, 3, 128)
    assert w.batch * w.nheads == 65535
    inp = make_inputs(w, 5)
    units = [0, 1, 7, 32767, 50000, 65534]
    print(f"case {w}: units {units}", flush=True)
    y, hT, ws, prob = _gpu_forward(inp, w, dev)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"],
                         units=units, chunk=w.chunk)
    u = ref["units"]
    b_idx, h_idx = u // w.nheads, u % w.nheads
    tol = TOL[w.dtype]
    check(np.stack([f64(y[b, :, h, :]) for b, h in zip(b_idx, h_idx)]), ref["y"], tol, "y (sampled units)")
    check(np.stack([f64(hT[b, h]) for b, h in zip(b_idx, h_idx)]), ref["hT"], tol, "hT (sampled units)")
    assert torch.isfinite(y.float()).all() and torch.isfinite(hT).all()


LARGEST = [
    # name, b, L, H, G, N, Q, sampled heads: L*H*P just below 2^30 (x rows), and
    # L*G*N just below 2^30 (B and C rows; one head per group, N = 512 column split)
    ("x_rows", 1, (1 << 30) // (32 * 64) - 1, 32, 1, 256, 256, [0, 31]),
    ("bc_rows", 1, (1 << 30) // (8 * 512) - 1, 8, 8, 512, 128, [0, 7]),
]


@pytest.mark.slow
@pytest.mark.parametrize("name,b,L,H,G,N,Q,units", LARGEST, ids=[c[0] for c in LARGEST])
def test_largest_sequence_sampled(name, b, L, H, G, N, Q, units):
    """The longest sequences the supported set allows along its two per-batch extents:
    the state pass addresses x and B rows with 32-bit byte offsets, which reach within a
    few KiB of 2^31 here (a ragged last chunk in both).  Sampled (batch, head) units
    against the oracle: y, hT and the chunk-start states."""
    dev = require_gpu()
    w = Workload(name, "bf16", b, L, H, 64, N, G, Q, has_h0=True)
    assert ssd.ssd_validate(ssd.make_problem(b, L, H, G, 64, N, Q, torch.bfloat16)) == 0
    assert ssd.ssd_validate(ssd.make_problem(b, L + 1, H, G, 64, N, Q, torch.bfloat16)) == 3
    print(f"case {w}: drawing inputs", flush=True)
    inp = make_inputs(w, 0)
    print("forward", flush=True)
    y, hT, ws, prob = _gpu_forward(inp, w, dev)
    del ws
    y_s = np.stack([f64(y[0, :, h, :]) for h in units])
    h_s = np.stack([f64(hT[0, h]) for h in units])
    assert torch.isfinite(y.float()).all() and torch.isfinite(hT).all()
    del y, hT
    print("stage states", flush=True)
    S, _ = _stage_states(inp, w, dev)
    S_s = np.stack([f64(S[0, h]) for h in units])
    del S
    torch.cuda.empty_cache()
    print("oracle", flush=True)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"],
                         units=units, chunk=w.chunk)
    tol = TOL["bf16"]
    check(y_s, ref["y"], tol, "y (sampled units)")
    check(h_s, ref["hT"], tol, "hT (sampled units)")
    check(S_s, ref["snaps"], tol, "chunk-start states (stage 2, sampled units)")
