"""Forward and decode step bound once (ForwardPlan, StepPlan), and the forward, the decode
step and the three stages recorded into HIP graphs.

The library allocates, clears and synchronises nothing inside its entry points, so they
can be captured on a side stream.  Every replay is compared bit for bit with the eager
call on the same inputs, with eager work (output poisoning, input refills) and
synchronisations between the replays; the refilled forward is also checked against the
oracle.
"""
import pytest
import torch

import oracle
import state_space_sequence_cumsum_amd as ssd
from state_space_sequence_cumsum_amd.inputs import Workload, make_inputs
from gpu_util import TOL, check, f64, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _wl(name, dtype, b, L, H, P, N, G, Q, h0=True):
    return Workload(name, dtype, b, L, H, P, N, G, Q, has_h0=h0)


PLAN_CASES = [
    _wl("plan_bf16_groups", "bf16", 1, 3000, 4, 64, 128, 1, 128),     # grouped state pass, ragged
    _wl("plan_bf16_n256", "bf16", 2, 1024, 8, 64, 256, 2, 256),
    _wl("plan_fp32", "fp32", 1, 256, 4, 64, 64, 1, 64, h0=False),
]


def _eager(d, w):
    y, hT = ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk)
    torch.cuda.synchronize()
    return y, hT


@pytest.mark.parametrize("w", PLAN_CASES, ids=[c.name for c in PLAN_CASES])
def test_forward_plan_matches_forward(w):
    dev = require_gpu()
    print(f"plan case {w}", flush=True)
    d = to_dev(make_inputs(w, 1), dev)
    y_ref, h_ref = _eager(d, w)
    plan = ssd.ForwardPlan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk)
    for _ in range(2):
        plan.y.fill_(float("nan"))
        plan.hT.fill_(float("nan"))
        y, hT = plan.run()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(hT, h_ref)


@pytest.mark.parametrize("w", PLAN_CASES, ids=[c.name for c in PLAN_CASES])
def test_forward_graph_replay(w):
    dev = require_gpu()
    print(f"graph case {w}", flush=True)
    inp = make_inputs(w, 2)
    d = to_dev(inp, dev)
    y_ref, h_ref = _eager(d, w)                     # also loads the kernels before capture
    side = torch.cuda.Stream(dev)
    plan = ssd.ForwardPlan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk,
                           stream=side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        plan.run()
    for k in range(4):
        plan.y.fill_(float("nan"))                  # eager work between the replays
        plan.hT.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.y, y_ref), f"replay {k}: y"
        assert torch.equal(plan.hT, h_ref), f"replay {k}: hT"
    # new values in the captured input tensors
    inp2 = make_inputs(w, 3)
    for k in ("x", "dt", "B", "C"):
        d[k].copy_(inp2[k].to(dev))
    if d["h0"] is not None:
        d["h0"].copy_(inp2["h0"].to(dev))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    y2, h2 = _eager(d, w)
    assert torch.equal(plan.y, y2) and torch.equal(plan.hT, h2)
    inp2["A"], inp2["D"] = inp["A"], inp["D"]       # A and D were not refilled
    ref = oracle.forward_full(inp2["x"], inp2["dt"], inp2["A"], inp2["B"], inp2["C"], inp2["D"],
                              inp2["h0"])
    check(f64(plan.y), ref["y"], TOL[w.dtype], "y after refill")
    check(f64(plan.hT), ref["hT"], TOL[w.dtype], "hT after refill")


def test_step_graph_replay():
    """A decode loop replaying one captured StepPlan.run(), its inputs refilled eagerly
    before each replay, matches ssd_step called eagerly token by token, bit for bit."""
    dev = require_gpu()
    w = _wl("step_graph", "bf16", 4, 12, 8, 64, 256, 2, 64)
    inp = make_inputs(w, 4)
    d = to_dev(inp, dev)
    b, H, P, G, N = w.batch, w.nheads, w.headdim, w.ngroups, w.dstate
    x = torch.empty(b, H, P, device=dev, dtype=torch.bfloat16)
    dt = torch.empty(b, H, device=dev, dtype=torch.bfloat16)
    B = torch.empty(b, G, N, device=dev, dtype=torch.bfloat16)
    C = torch.empty_like(B)
    h_graph = d["h0"].clone()
    h_call = d["h0"].clone()

    def refill(t):
        x.copy_(d["x"][:, t]); dt.copy_(d["dt"][:, t]); B.copy_(d["B"][:, t]); C.copy_(d["C"][:, t])

    refill(0)
    y_warm = ssd.ssd_step(x, dt, d["A"], B, C, d["D"], d["h0"].clone())   # kernels loaded
    torch.cuda.synchronize()
    side = torch.cuda.Stream(dev)
    plan = ssd.StepPlan(x, dt, d["A"], B, C, d["D"], h_graph, stream=side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        plan.run()
    torch.cuda.synchronize()
    assert torch.equal(h_graph, d["h0"])            # capture ran nothing
    for t in range(w.seqlen):
        refill(t)
        plan.y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        y_call = ssd.ssd_step(d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(), d["A"],
                              d["B"][:, t].contiguous(), d["C"][:, t].contiguous(), d["D"], h_call)
        torch.cuda.synchronize()
        assert torch.equal(plan.y, y_call), t
    assert torch.equal(h_graph, h_call)
    del y_warm
    ref = oracle.forward_full(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"])
    check(f64(h_graph), ref["hT"], TOL["bf16"], "state after the replays")


def test_stages_graph_replay():
    """The three stage entry points recorded into one graph on a side stream, with every
    intermediate preallocated, replay to the eager stages' outputs bit for bit."""
    dev = require_gpu()
    w = _wl("stages_graph", "bf16", 2, 1280, 4, 64, 128, 2, 64)
    d = to_dev(make_inputs(w, 11), dev)
    prob = ssd.problem_of(d["x"], d["B"], w.chunk)
    G2, dtT = ssd.ssd_chunk_cumsum(prob, d["dt"], d["A"])
    S, hT = ssd.ssd_state_pass(prob, d["x"], d["B"], G2, dtT, d["h0"])
    y = ssd.ssd_chunk_out(prob, d["x"], d["B"], d["C"], G2, dtT, S, d["D"])
    torch.cuda.synchronize()
    outs = {"G2": G2, "dtT": dtT, "S": S, "hT": hT, "y": y}
    ref = {k: v.clone() for k, v in outs.items()}
    side = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        ssd.ssd_chunk_cumsum(prob, d["dt"], d["A"], G2, dtT, stream=side)
        ssd.ssd_state_pass(prob, d["x"], d["B"], G2, dtT, d["h0"], S=S, hT=hT, stream=side)
        ssd.ssd_chunk_out(prob, d["x"], d["B"], d["C"], G2, dtT, S, d["D"], y=y, stream=side)
    for k in range(3):
        for t in outs.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in outs.items():
            assert torch.equal(t, ref[name]), f"replay {k}: {name}"
