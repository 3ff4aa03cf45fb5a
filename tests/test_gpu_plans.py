"""Every launch configuration of the forward's search space (ssd_plan_candidates) against the
oracle, and the per-shape search (autotune) that picks among them.

The kernels differ per candidate (state columns per workgroup, B transposed in registers
or through LDS, chains split into 1 .. nc groups with the group scan and the carried-state
correction, head-blocked or one-head chunk output), so every candidate's forward is checked
against the fp64 oracle within the bound of its precision, and against the default plan's
forward.  Some shapes scale A down so that the decay over a group of chunks stays near one
and the carried state is most of each chunk-start state.
"""
import numpy as np
import pytest
import torch

import oracle
import state_space_sequence_cumsum_amd as ssd
from gpu_util import TOL, check, check_dev, f64, require_gpu, to_dev
from state_space_sequence_cumsum_amd.inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _wl(name, dtype, b, L, H, N, G, Q, h0=True):
    return Workload(name, dtype, b, L, H, 64, N, G, Q, has_h0=h0)


# (workload, A scale)
SHAPES = [
    (_wl("p_n256_q128_g2", "bf16", 1, 700, 4, 256, 2, 128), 1e-2),     # ragged, head-blocked
    (_wl("p_n512_q128", "bf16", 2, 520, 2, 512, 1, 128), 1.0),          # ragged, column halves
    (_wl("p_n128_q256", "bf16", 1, 600, 4, 128, 1, 256, h0=False), 1e-2),
    (_wl("p_n64_q64", "bf16", 1, 512, 2, 64, 1, 64), 1.0),              # one-head output only
    (_wl("p_n256_q256", "bf16", 1, 1024, 8, 256, 2, 256), 1e-2),        # 4 heads per group
    (_wl("p_n384_q128", "bf16", 1, 384, 2, 384, 1, 128), 1.0),          # 128 / 64 columns
    (_wl("p_n256_q64", "bf16", 1, 330, 2, 256, 1, 64), 1e-2),           # one sub-step per chunk
    (_wl("p_fp32_q64", "fp32", 1, 300, 2, 128, 1, 64), 1e-2),
]


def _inputs(w, scale, seed=21):
    inp = make_inputs(w, seed)
    inp["A"].mul_(scale)
    return inp


@pytest.mark.parametrize("w,scale", SHAPES, ids=[w.name for w, _ in SHAPES])
def test_every_candidate_plan(w, scale):
    dev = require_gpu()
    inp = _inputs(w, scale)
    d = to_dev(inp, dev)
    prob = ssd.problem_of(d["x"], d["B"], w.chunk)
    cands = ssd.plan_candidates(prob)
    print(f"case {w.name}: {len(cands)} candidate plans", flush=True)
    ref = oracle.forward_full(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                              inp["h0"], chunk=w.chunk)
    tol = TOL[w.dtype]
    y0, h0T = ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                              chunk=w.chunk)
    torch.cuda.synchronize()
    worst = 0.0
    for i, c in enumerate(cands):
        print(f"  plan {i}: {c}", flush=True)
        ws = ssd.workspace_for(prob, dev, c)
        y = torch.full_like(y0, float("nan"))
        hT = torch.full_like(h0T, float("nan"))
        ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk,
                        y=y, hT=hT, workspace=ws, launch_plan=c)
        torch.cuda.synchronize()
        worst = max(worst, check(f64(y), ref["y"], tol, f"y, plan {i}"))
        check(f64(hT), ref["hT"], tol, f"hT, plan {i}")
        check_dev(y, y0, tol, f"y, plan {i} against the default plan")
        if i == 0:   # the default plan through ssd_forward_planned is ssd_forward itself
            assert torch.equal(y, y0) and torch.equal(hT, h0T)
    print(f"  worst y error over the plans: {worst:.3e}", flush=True)


def test_planned_stages_match_planned_forward():
    """Stages 0..3 one at a time under a non-default plan (ForwardPlan.run_stage) give the
    forward's results bit for bit."""
    dev = require_gpu()
    w, scale = SHAPES[0]
    d = to_dev(_inputs(w, scale), dev)
    prob = ssd.problem_of(d["x"], d["B"], w.chunk)
    default = ssd.ssd_plan(prob)
    other = [c for c in ssd.plan_candidates(prob)
             if c["sp_groups"] > 1 and c["sp_columns"] != default["sp_columns"]][0]
    plan = ssd.ForwardPlan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                           chunk=w.chunk, launch_plan=other)
    assert plan.launch_plan == other
    y, hT = plan.run()
    torch.cuda.synchronize()
    y_ref, h_ref = y.clone(), hT.clone()
    y.fill_(float("nan"))
    hT.fill_(float("nan"))
    for stage in range(4):
        plan.run_stage(stage)
    torch.cuda.synchronize()
    assert torch.equal(plan.y, y_ref) and torch.equal(plan.hT, h_ref)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(ssd.FORWARD_EVENTS)]
    for e in ev:
        e.record()
    plan.run_timed(ev)
    torch.cuda.synchronize()
    assert torch.equal(plan.y, y_ref)
    assert all(ev[i].elapsed_time(ev[i + 1]) >= 0 for i in range(len(ev) - 1))


@pytest.mark.parametrize("w,scale", [SHAPES[0], SHAPES[3]], ids=[SHAPES[0][0].name, SHAPES[3][0].name])
def test_autotune_picks_a_candidate(w, scale):
    dev = require_gpu()
    inp = _inputs(w, scale)
    d = to_dev(inp, dev)
    prob = ssd.problem_of(d["x"], d["B"], w.chunk)
    res = ssd.autotune(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk,
                       reps=5, warmup=1)
    print(f"case {w.name}: {res['plan']} {res['forward_us']} us (default {res['default_forward_us']} us)",
          flush=True)
    cands = ssd.plan_candidates(prob)
    assert res["plan"] in cands and res["default_plan"] == cands[0]
    assert res["forward_us"] <= res["default_forward_us"]
    assert len(res["state_pass"]) >= 2 and res["chunk_out"]
    y, hT = ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk,
                            launch_plan=res["plan"])
    torch.cuda.synchronize()
    ref = oracle.forward_full(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                              inp["h0"], chunk=w.chunk)
    check(f64(y), ref["y"], TOL[w.dtype], "y under the tuned plan")
    check(f64(hT), ref["hT"], TOL[w.dtype], "hT under the tuned plan")
    assert np.isfinite(f64(y)).all()


# the one-launch forward (fp32, 64-token chunks, dstate 64, at most 8 chunks)
FUSED = [
    (_wl("fused_8chunks", "fp32", 2, 512, 3, 64, 1, 64), 1.0),          # the longest chain
    (_wl("fused_g2_ragged", "fp32", 1, 450, 4, 64, 2, 64), 1e-2),       # ragged, 2 B/C groups
    (_wl("fused_one_chunk", "fp32", 3, 40, 2, 64, 1, 64, h0=False), 1.0),  # one partial chunk
    (_wl("fused_5chunks_ragged", "fp32", 1, 300, 5, 64, 1, 64), 1.0),   # a ring refill, ragged
    (_wl("fused_many_heads", "fp32", 6, 150, 64, 64, 4, 64), 1.0),      # 2304 workgroups, 4 groups
]


@pytest.mark.parametrize("w,scale", FUSED, ids=[w.name for w, _ in FUSED])
def test_one_launch_forward(w, scale):
    """The one-launch plan against the oracle and against the general four-launch path,
    with and without the final state; the stage-1 values it leaves in the workspace equal
    ssd_chunk_cumsum's bit for bit."""
    dev = require_gpu()
    inp = _inputs(w, scale)
    d = to_dev(inp, dev)
    prob = ssd.problem_of(d["x"], d["B"], w.chunk)
    plan = ssd.ssd_plan(prob)
    assert plan["fused"] == 1
    print(f"case {w.name}: {plan}", flush=True)
    ws = ssd.workspace_for(prob, dev)
    ws.fill_(0xFF)
    y, hT = ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                            chunk=w.chunk, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.forward_full(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                              inp["h0"], chunk=w.chunk)
    tol = TOL[w.dtype]
    check(f64(y), ref["y"], tol, "y (one launch)")
    check(f64(hT), ref["hT"], tol, "hT (one launch)")
    G2, dtT = ssd.ssd_chunk_cumsum(prob, d["dt"], d["A"])
    torch.cuda.synchronize()
    v = ssd.workspace_views(prob, ws)
    assert torch.equal(v["G2"], G2) and torch.equal(v["dtT"], dtT)
    general = [c for c in ssd.plan_candidates(prob) if not c["fused"]][0]
    y2, h2 = ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                             chunk=w.chunk, launch_plan=general)
    torch.cuda.synchronize()
    check_dev(y, y2, tol, "y: one launch against the general path")
    check_dev(hT, h2, tol, "hT: one launch against the general path")
    y3 = torch.full_like(y, float("nan"))
    ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk,
                    y=y3, want_final=False)
    torch.cuda.synchronize()
    assert torch.equal(y3, y)


@pytest.mark.parametrize("w", [
    _wl("inplace_one_launch", "fp32", 2, 512, 3, 64, 1, 64),      # the one-launch plan's shape
    _wl("inplace_bf16_grouped", "bf16", 1, 3000, 4, 128, 1, 128),  # grouped state pass and scan
], ids=lambda w: w.name)
def test_in_place_final_state(w):
    """h0 and hT the same buffer (the boundary allows it): the final state replaces the
    initial one in place and y is unchanged.  For the one-launch shape the call runs the
    four-launch plan of one serial chain instead, whose workgroups each read their own
    slice of h0 before writing it."""
    dev = require_gpu()
    inp = _inputs(w, 1.0)
    d = to_dev(inp, dev)
    prob = ssd.problem_of(d["x"], d["B"], w.chunk)
    print(f"case {w.name}: {ssd.ssd_plan(prob)}", flush=True)
    h = d["h0"].clone()
    y, hT = ssd.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], h, chunk=w.chunk,
                            hT=h)
    torch.cuda.synchronize()
    assert hT.data_ptr() == h.data_ptr()
    ref = oracle.forward_full(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                              inp["h0"], chunk=w.chunk)
    check(f64(y), ref["y"], TOL[w.dtype], "y (h0 and hT one buffer)")
    check(f64(h), ref["hT"], TOL[w.dtype], "hT in place")
