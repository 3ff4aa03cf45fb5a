"""Per-shape search over the forward pass's launch configurations.

The dbyun.net page chooses its kernels' optimisations per shape together with block
size and occupancy, by timing every combination on the device (section "Mamba-2
性能优化"; the thetimeai.ru page, section "Почему раскладка памяти важна не меньше
формул", says the same of its search).  Here the search space is the list that
ssd_plan_candidates returns for the problem: the state-pass kernel (state columns per
workgroup, B transposed in registers or through LDS), the split of each chain of chunks
into groups, and the chunk-output kernel (heads per workgroup, or one head).

The state pass and its group scan depend only on the state-pass kernel and the grouping,
and the chunk output only on its own kernel and on whether the state pass is grouped, so
the search runs in two passes instead of over the product:

1. every distinct (state-pass kernel, grouping), each with the chunk-output choice of
   the cost model (or the first one the candidates pair with it): stage 1 then stage 2
   (state pass, group scan) launched back to back ``reps`` times between one event pair;
2. with the fastest of pass 1, every chunk-output choice: stage 3 alone ``reps`` times.

The winner of both passes and the cost model's plan are then timed as whole forwards and
the faster is returned, so the search never returns a plan slower than the default by
its own measurement.  Every launch goes through the C ABI (ssd_forward_planned); this
module only orders the calls and reads the events.
"""
from __future__ import annotations

import statistics

import torch

from .binding import ForwardPlan, plan_candidates, problem_of, ssd_workspace_bytes_planned

SP_KEYS = ("sp_columns", "sp_register_transposed", "sp_group_chunks", "sp_groups")
CO_KEYS = ("co_head_blocked", "co_heads_per_block")


def _time(fn, reps: int, stream, batches: int = 3) -> float:
    """Median over `batches` of (event time of `reps` back-to-back calls of fn) / reps, in
    microseconds."""
    out = []
    for _ in range(batches):
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        z.record(stream)
        z.synchronize()
        out.append(a.elapsed_time(z) * 1e3 / reps)
    return statistics.median(out)


def autotune(x, dt, A, B, C, D, h0=None, *, chunk: int, reps: int = 20, warmup: int = 3,
             stream=None, max_workspace_bytes: int = 4 << 30) -> dict:
    """Search the launch configurations of ssd_forward for these inputs' shape.

    Returns a dict with ``plan`` (the chosen candidate, a field-name dict to pass as
    ``launch_plan``), ``default_plan`` (ssd_plan's choice), ``forward_us`` and
    ``default_forward_us`` (whole forwards under each, event-timed), and the two passes'
    tables ``state_pass`` and ``chunk_out`` (the varied fields and the microseconds per
    launch).  Candidates whose workspace exceeds ``max_workspace_bytes`` are skipped.
    The inputs are only read; outputs go to scratch tensors.
    """
    dev = x.device
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    problem = problem_of(x, B, chunk)
    cands = plan_candidates(problem)
    default = cands[0]
    cands = [c for c in cands if ssd_workspace_bytes_planned(problem, c) <= max_workspace_bytes]
    if not cands:
        cands = [default]
    ws = torch.empty(max(ssd_workspace_bytes_planned(problem, c) for c in cands + [default]),
                     device=dev, dtype=torch.uint8)
    y = torch.empty_like(x)
    b, H, P, N = x.shape[0], x.shape[2], x.shape[3], B.shape[3]
    hT = torch.empty(b, H, P, N, device=dev, dtype=torch.float32)

    def plan_for(c):
        return ForwardPlan(x, dt, A, B, C, D, h0, chunk=chunk, y=y, hT=hT, workspace=ws,
                           stream=stream, launch_plan=c)

    def pair(p):
        p.run_stage(1)
        p.run_stage(2)

    # pass 1: state pass + group scan per (kernel, grouping)
    sp_table, seen = [], {}
    for c in cands:
        key = tuple(c[k] for k in SP_KEYS)
        prefer = tuple(c[k] for k in CO_KEYS) == tuple(default[k] for k in CO_KEYS)
        if key not in seen or prefer:
            seen[key] = c
    for key, c in seen.items():
        p = plan_for(c)
        p.run_stage(0)
        for _ in range(warmup):
            pair(p)
        us = _time(lambda: pair(p), reps, stream)
        sp_table.append({**{k: c[k] for k in SP_KEYS}, "us": round(us, 3)})
    best_sp = min(sp_table, key=lambda r: r["us"])

    # pass 2: chunk output per kernel choice, with the best state pass
    co_table = []
    for c in cands:
        if any(c[k] != best_sp[k] for k in SP_KEYS):
            continue
        p = plan_for(c)
        p.run()                      # the workspace as a forward under this plan leaves it
        for _ in range(warmup):
            p.run_stage(3)
        us = _time(lambda: p.run_stage(3), reps, stream)
        co_table.append({**{k: c[k] for k in CO_KEYS}, "us": round(us, 3), "_plan": c})
    best = min(co_table, key=lambda r: r["us"])["_plan"]

    # whole forwards: the search's winner against the cost model's plan
    fwd = {}
    for name, c in (("tuned", best), ("default", default)):
        p = plan_for(c)
        for _ in range(warmup):
            p.run()
        fwd[name] = _time(p.run, reps, stream)
    chosen = best if fwd["tuned"] < fwd["default"] else default
    torch.cuda.synchronize(dev)
    del ws
    return {"plan": chosen, "default_plan": default,
            "forward_us": round(min(fwd["tuned"], fwd["default"]), 3),
            "default_forward_us": round(fwd["default"], 3),
            "candidates": len(cands),
            "state_pass": sp_table,
            "chunk_out": [{k: v for k, v in r.items() if k != "_plan"} for r in co_table]}
