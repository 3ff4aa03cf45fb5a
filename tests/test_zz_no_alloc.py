"""ssd_forward_noalloc (static device scratch, no allocation) against ssd_forward.

Both entry points run the same kernels, so on identical inputs their outputs must
agree bit for bit (and so meet the parity bar of the forward itself).  The scratch
keeps the previous call's contents, so the calls come in a row, the second on a
smaller problem, and then from a HIP graph replayed several times.
"""
import ctypes

import pytest
import torch

import oracle
import state_space_sequence_cumsum_amd as ssd
from state_space_sequence_cumsum_amd.inputs import WORKLOADS, Workload, make_inputs
from gpu_util import TOL, check, f64, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _pair(w, seed, dev, stream=None):
    """(y, hT) from ssd_forward_noalloc and from ssd_forward, same inputs."""
    d = to_dev(make_inputs(w, seed), dev)
    io = d["x"].dtype
    outs = []
    for fn in ("noalloc", "forward"):
        y = torch.full((w.batch, w.seqlen, w.nheads, w.headdim), float("nan"), device=dev, dtype=io)
        hT = torch.full((w.batch, w.nheads, w.headdim, w.dstate), float("nan"), device=dev,
                        dtype=torch.float32)
        args = (d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"])
        if fn == "noalloc":
            ssd.ssd_forward_noalloc(*args, chunk=w.chunk, y=y, hT=hT, stream=stream)
        else:
            ssd.ssd_forward(*args, chunk=w.chunk, y=y, hT=hT, stream=stream)
        outs.append((y, hT))
    torch.cuda.synchronize()
    return d, outs


# the largest workload that fits the scratch first, then smaller ones (fp32, ragged and
# grouped with a one-head tail, one serial group), each reusing what the previous left
ROW = [
    WORKLOADS["bf16_b1_L16384_H32_P64_N256_Q256"],
    WORKLOADS["bf16_b2_L2048_H24_P64_N128_Q256"],
    Workload("ragged_groups", "bf16", 1, 3000, 4, 64, 128, 1, 128, has_h0=True),
    WORKLOADS["fp32_b1_L256_H4_P64_N64_Q64"],
]


def test_noalloc_calls_in_a_row_match_forward():
    dev = require_gpu()
    prob = None
    for k, w in enumerate(ROW):
        p = ssd.make_problem(w.batch, w.seqlen, w.nheads, w.ngroups, w.headdim, w.dstate,
                             w.chunk, w.dtype)
        assert 0 < ssd.ssd_workspace_bytes(p) <= ssd.binding.SCRATCH_BYTES, w.name
        if k > 0:
            assert ssd.ssd_workspace_bytes(p) < ssd.ssd_workspace_bytes(prob), "second call is smaller"
        prob = p
        print(f"case {w.name} (call {k + 1} in a row)", flush=True)
        d, ((y1, h1), (y2, h2)) = _pair(w, 20 + k, dev)
        assert torch.equal(y1, y2) and torch.equal(h1, h2), w.name
        check(f64(y1), f64(y2), TOL[w.dtype], "y against ssd_forward")
        check(f64(h1), f64(h2), TOL[w.dtype], "hT against ssd_forward")


def test_noalloc_smallest_case_against_oracle():
    """The last, smallest call of a row (after a larger one) against the oracle itself."""
    dev = require_gpu()
    _pair(ROW[0], 1, dev)
    w = Workload("small_after_large", "bf16", 2, 700, 4, 64, 64, 2, 64, has_h0=True)
    inp = make_inputs(w, 3)
    d = to_dev(inp, dev)
    y, hT = ssd.ssd_forward_noalloc(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                                    chunk=w.chunk)
    torch.cuda.synchronize()
    ref = oracle.forward_full(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"])
    check(f64(y), ref["y"], TOL["bf16"], "y against the oracle")
    check(f64(hT), ref["hT"], TOL["bf16"], "hT against the oracle")


def test_noalloc_on_a_side_stream():
    dev = require_gpu()
    side = torch.cuda.Stream(dev)
    w = ROW[1]
    d, ((y1, h1), (y2, h2)) = _pair(w, 7, dev, stream=side)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_noalloc_graph_replays():
    """Recorded into a HIP graph (the call allocates nothing), replayed with eager work and
    synchronisations between the replays; every replay equals the eager forward."""
    dev = require_gpu()
    w = ROW[2]
    d = to_dev(make_inputs(w, 11), dev)
    io = d["x"].dtype
    y = torch.empty(w.batch, w.seqlen, w.nheads, w.headdim, device=dev, dtype=io)
    hT = torch.empty(w.batch, w.nheads, w.headdim, w.dstate, device=dev, dtype=torch.float32)
    args = (d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"])
    y_ref, h_ref = ssd.ssd_forward(*args, chunk=w.chunk)
    side = torch.cuda.Stream(dev)
    ssd.ssd_forward_noalloc(*args, chunk=w.chunk, y=y, hT=hT, stream=side)   # address looked up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        ssd.ssd_forward_noalloc(*args, chunk=w.chunk, y=y, hT=hT, stream=side)
    for rep in range(4):
        y.fill_(float("nan"))
        hT.fill_(float("nan"))
        ssd.ssd_forward(*args, chunk=w.chunk)      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(hT, h_ref), f"replay {rep}"


def test_noalloc_rejects_too_large_before_launch():
    dev = require_gpu()
    w = WORKLOADS["bf16_b1_L65536_H32_P64_N512_Q128"]
    p = ssd.make_problem(w.batch, w.seqlen, w.nheads, w.ngroups, w.headdim, w.dstate, w.chunk,
                         w.dtype)
    assert ssd.ssd_workspace_bytes(p) > ssd.binding.SCRATCH_BYTES
    x = torch.zeros(1, 128, 32, 64, device=dev, dtype=torch.bfloat16)   # never read
    lib = ssd.binding.lib()
    ok = x.data_ptr()
    assert lib.ssd_forward_noalloc(ctypes.byref(p), ok, ok, ok, ok, ok, ok, None, ok, None,
                                   None) == 7
    assert lib.ssd_last_hip_error() == 0
