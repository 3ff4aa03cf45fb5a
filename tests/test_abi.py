"""Host-side checks of the C ABI: the library loads, exports what include/ssd.h
declares, and validates arguments before any launch.  No GPU needed."""
import ctypes

import pytest
import torch

import state_space_sequence_cumsum_amd as ssd
from state_space_sequence_cumsum_amd import binding


def test_library_exports_every_declared_symbol():
    names = binding.header_functions()
    assert {"ssd_chunk_cumsum", "ssd_state_pass", "ssd_chunk_out", "ssd_forward",
            "ssd_step"} <= set(names)
    lib = binding.lib()
    for n in names:
        assert hasattr(lib, n), f"libssd.so does not export {n}"


def _p(**kw):
    base = dict(batch=1, seqlen=16384, nheads=32, ngroups=1, headdim=64, dstate=256, chunk=256,
                dtype="bf16")
    base.update(kw)
    return ssd.make_problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(dtype="fp32", dstate=64, chunk=64), 0),
    (dict(seqlen=1), 0),
    (dict(seqlen=1000, chunk=128, dstate=512), 0),
    (dict(nheads=16, ngroups=2), 0),
    (dict(batch=0), 2),
    (dict(seqlen=-1), 2),
    (dict(nheads=6, ngroups=4), 2),
    (dict(chunk=0), 2),
    (dict(headdim=128), 3),
    (dict(dstate=96), 3),
    (dict(dstate=1024), 3),
    (dict(chunk=32), 3),
    (dict(dtype=7), 3),
])
def test_validate(kw, status):
    assert ssd.ssd_validate(_p(**kw)) == status


def test_validate_null_problem():
    assert binding.lib().ssd_validate(None) == 1


def test_workspace_size_and_layout():
    p = _p()
    g2, dtt, s = ssd.ssd_workspace_layout(p)
    cum = 1 * 32 * 64 * 256 * 4          # b*H*Lp fp32
    snap = 1 * 32 * 64 * 64 * 256 * 2    # b*H*nc*P*N bf16
    # G2, dtT, the forward's own state-pass weights, then S
    assert (g2, dtt, s) == (0, cum, 3 * cum)
    # plus the grouped state pass's scratch: group states, group and chunk decays
    assert ssd.ssd_workspace_bytes(p) >= 3 * cum + snap
    assert all(o % 256 == 0 for o in (g2, dtt, s))
    # ragged length: padded to whole chunks, fp32 snapshots for fp32 problems
    q = _p(seqlen=1000, chunk=128, dtype="fp32", dstate=64)
    nc = 8
    g2, dtt, s = ssd.ssd_workspace_layout(q)
    assert dtt >= 32 * nc * 128 * 4 and dtt % 256 == 0 and s >= 3 * dtt
    assert ssd.ssd_workspace_bytes(q) >= s + 32 * nc * 64 * 64 * 4
    assert ssd.ssd_workspace_bytes(_p(dstate=100)) == 0


def test_entry_points_reject_bad_arguments_without_launching():
    lib = binding.lib()
    p = _p()
    fake = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    # missing pointers
    assert lib.ssd_chunk_cumsum(ctypes.byref(p), None, fake, fake, fake, None) == 1
    assert lib.ssd_chunk_cumsum(ctypes.byref(p), fake, fake, fake, None, None) == 1
    assert lib.ssd_state_pass(ctypes.byref(p), fake, None, fake, fake, None, fake, None, None) == 1
    assert lib.ssd_chunk_out(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, fake, None) == 1
    assert lib.ssd_forward(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None, None,
                           fake, 10**12, None) == 1
    # workspace too small or missing
    assert lib.ssd_forward(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, fake, None,
                           fake, 100, None) == 4
    assert lib.ssd_forward(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, fake, None,
                           None, 10**12, None) == 4
    # bad shapes win over everything
    bad = _p(nheads=6, ngroups=4)
    assert lib.ssd_forward(ctypes.byref(bad), None, None, None, None, None, None, None, None,
                           None, None, 0, None) == 2
    # timed forward: events array with a NULL handle
    ev = (ctypes.c_void_p * binding.FORWARD_EVENTS)(fake.value, fake.value, fake.value, None,
                                                     fake.value)
    assert lib.ssd_forward_timed(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, fake,
                                 None, fake, 10**12, None, ev) == 1
    assert lib.ssd_last_hip_error() == 0


def test_forward_stage_validates_before_launching():
    lib = binding.lib()
    p = _p()
    fake = ctypes.c_void_p(256)
    args = [fake] * 6 + [None, fake, None, fake]   # x dt A B C D h0 y hT workspace
    for stage in (-1, 4):
        assert lib.ssd_forward_stage(ctypes.byref(p), *args, 10**12, stage, None) == 3
    assert lib.ssd_forward_stage(ctypes.byref(p), *args, 100, 3, None) == 4
    no_y = [fake] * 6 + [None, None, None, fake]
    assert lib.ssd_forward_stage(ctypes.byref(p), *no_y, 10**12, 0, None) == 1
    bad = _p(nheads=6, ngroups=4)
    assert lib.ssd_forward_stage(ctypes.byref(bad), *args, 10**12, 7, None) == 2
    assert lib.ssd_last_hip_error() == 0


def test_misaligned_pointers_are_rejected_without_launching():
    lib = binding.lib()
    p = _p()
    ok = ctypes.c_void_p(4096)
    off = ctypes.c_void_p(4096 + 8)   # element-aligned, not on 16 bytes
    assert lib.ssd_chunk_cumsum(ctypes.byref(p), off, ok, ok, off, None) == 6
    assert lib.ssd_state_pass(ctypes.byref(p), off, ok, ok, ok, None, ok, None, None) == 6
    assert lib.ssd_state_pass(ctypes.byref(p), ok, ok, ok, ok, off, ok, None, None) == 6
    assert lib.ssd_chunk_out(ctypes.byref(p), ok, ok, ok, ok, ok, ok, ok, off, None) == 6
    assert lib.ssd_forward(ctypes.byref(p), ok, ok, ok, ok, ok, ok, None, ok, None, off, 10**12,
                           None) == 6
    assert lib.ssd_forward(ctypes.byref(p), ok, ok, ok, off, ok, ok, None, ok, None, ok, 10**12,
                           None) == 6
    sp = _p(seqlen=1)
    assert lib.ssd_step(ctypes.byref(sp), ok, off, off, ok, ok, off, off, ok, None) == 6
    assert lib.ssd_last_hip_error() == 0


def _sp(**kw):
    base = dict(batch=4, seqlen=1, nheads=32, ngroups=1, headdim=64, dstate=256, chunk=0,
                dtype="bf16")
    base.update(kw)
    return ssd.make_problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(), 1),                       # valid shape: reaches the NULL-pointer check
    (dict(dstate=512, headdim=7, dtype="fp32", nheads=6, ngroups=3), 1),
    (dict(seqlen=2), 2),
    (dict(seqlen=0), 2),
    (dict(batch=0), 2),
    (dict(nheads=6, ngroups=4), 2),
    (dict(dstate=96), 3),
    (dict(dstate=576), 3),
    (dict(dtype=9), 3),
    (dict(batch=1 << 20, nheads=1 << 12, headdim=64), 3),
    # the dispatch grid: b * H * ceil(P / 4) waves in workgroups of 4 waves, at most
    # 2^24 - 1 workgroups (2^32 work-items); within the 2^31 row-index limit
    (dict(batch=1 << 24, nheads=4, headdim=1, dstate=64), 3),          # 2^26 waves
    (dict(batch=(1 << 24) - 1, nheads=4, headdim=1, dstate=64), 1),    # 2^26 - 4 waves
    (dict(batch=1 << 22, nheads=4, headdim=13, dstate=64), 3),         # ceil(13/4) = 4 rows
    (dict(batch=(1 << 22) - 1, nheads=4, headdim=13, dstate=64), 1),
])
def test_step_validates_before_launching(kw, status):
    lib = binding.lib()
    p = _sp(**kw)
    ok = ctypes.c_void_p(4096)
    # every pointer given except y: a valid problem stops at SSD_ERR_NULL_ARG
    assert lib.ssd_step(ctypes.byref(p), ok, ok, ok, ok, ok, ok, ok, None, None) == status
    assert lib.ssd_step(None, ok, ok, ok, ok, ok, ok, ok, ok, None) == 1


def test_status_strings():
    for s in range(9):
        assert ssd.ssd_status_string(s)
    assert "unknown" in ssd.ssd_status_string(42)


def test_noalloc_scratch_limit_checked_before_launching():
    """ssd_forward_noalloc refuses shapes whose workspace exceeds its static scratch, and bad
    shapes, on the host (no pointer is touched, no GPU is needed)."""
    lib = binding.lib()
    text = open(binding.HEADER).read()
    assert "#define SSD_SCRATCH_BYTES (128u << 20)" in text
    assert binding.SCRATCH_BYTES == 128 << 20
    fake = ctypes.c_void_p(4096)
    big = _p(seqlen=65536, dstate=512, chunk=128)
    assert ssd.ssd_workspace_bytes(big) > binding.SCRATCH_BYTES
    assert lib.ssd_forward_noalloc(ctypes.byref(big), fake, fake, fake, fake, fake, fake, None,
                                   fake, None, None) == 7
    bad = _p(nheads=6, ngroups=4)
    assert lib.ssd_forward_noalloc(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, None,
                                   fake, None, None) == 2
    assert lib.ssd_forward_noalloc(None, fake, fake, fake, fake, fake, fake, None, fake, None,
                                   None) == 1
    # the headline forward fits
    assert 0 < ssd.ssd_workspace_bytes(_p(seqlen=16384, dstate=256, chunk=256)) <= binding.SCRATCH_BYTES
    assert lib.ssd_last_hip_error() == 0


def test_binding_refuses_host_tensors():
    x = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16)
    B = torch.zeros(1, 64, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ssd.ssd_forward(x, torch.zeros(1, 64, 2, dtype=torch.bfloat16), torch.zeros(2), B, B,
                        torch.zeros(2), chunk=64)
    # the plans check their tensors when they are made, before any call
    with pytest.raises(ValueError):
        ssd.ForwardPlan(x, torch.zeros(1, 64, 2, dtype=torch.bfloat16), torch.zeros(2), B, B,
                        torch.zeros(2), chunk=64)
    with pytest.raises(ValueError):
        ssd.StepPlan(torch.zeros(1, 2, 64, dtype=torch.bfloat16), torch.zeros(1, 2, dtype=torch.bfloat16),
                     torch.zeros(2), torch.zeros(1, 1, 64, dtype=torch.bfloat16),
                     torch.zeros(1, 1, 64, dtype=torch.bfloat16), torch.zeros(2), torch.zeros(1, 2, 64, 64))


def test_launch_plan_per_shape():
    """ssd_plan reports the per-shape launch choices (host only)."""
    # headline: 8 groups of 8 chunks, one state-pass workgroup per CU, 8 heads per
    # head-blocked chunk-output workgroup of 2 Q threads
    assert ssd.ssd_plan(_p(seqlen=16384, nheads=32, dstate=256, chunk=256)) == dict(
        sp_group_chunks=8, sp_groups=8, sp_columns=256, sp_workgroups=256, scan=1,
        co_head_blocked=1, co_heads_per_block=8, co_column_split=1, co_workgroups=256,
        co_threads=512, sp_register_transposed=0, sp_threads=512, fused=0)
    # N = 512 with 128-token chunks: the register-transposed state pass, two 256-column
    # workgroups of 4 waves per chain and two per CU (8 groups of 64 chunks), the chunk
    # output's columns split over wave pairs
    p512 = ssd.ssd_plan(_p(seqlen=65536, dstate=512, chunk=128))
    assert (p512["sp_columns"], p512["sp_groups"], p512["co_column_split"], p512["co_threads"]) == (256, 8, 2, 512)
    assert (p512["sp_register_transposed"], p512["sp_threads"]) == (1, 256)
    assert p512["sp_workgroups"] == 32 * 2 * 8 and p512["co_workgroups"] == 512 * (32 // p512["co_heads_per_block"])
    # below 512 state columns the LDS-transposed state pass
    for n in (64, 128, 256, 384, 448):
        assert ssd.ssd_plan(_p(dstate=n, chunk=128))["sp_register_transposed"] == 0
    # ragged: 23 full chunks head-blocked (one head per block here) plus the last chunk of
    # each (batch, head) on the one-head kernel
    pr = ssd.ssd_plan(_p(seqlen=3000, nheads=2, dstate=128, chunk=128))
    assert pr["co_head_blocked"] == 1 and pr["co_heads_per_block"] == 1
    assert pr["co_workgroups"] == 23 * 2 + 2
    # 64-token chunks and N = 384 use the one-head kernel
    for kw in (dict(chunk=64), dict(dstate=384, chunk=128)):
        q = ssd.ssd_plan(_p(**kw))
        assert q["co_head_blocked"] == 0 and q["co_heads_per_block"] == 1
    # fp32 with at most 8 chunks of 64 tokens and dstate 64: the whole forward as one launch,
    # one 256-thread workgroup per (batch, head, chunk or final state, half of the headdim)
    f0 = ssd.ssd_plan(_p(seqlen=256, nheads=4, dstate=64, chunk=64, dtype="fp32"))
    assert (f0["fused"], f0["co_workgroups"], f0["co_threads"], f0["sp_workgroups"], f0["scan"]) == (1, 40, 256, 0, 0)
    assert ssd.ssd_plan(_p(seqlen=512, nheads=4, dstate=64, chunk=64, dtype="fp32"))["fused"] == 1
    for kw in (dict(seqlen=513), dict(dstate=128), dict(chunk=128), dict(dtype="bf16")):
        args = dict(seqlen=256, nheads=4, dstate=64, chunk=64, dtype="fp32")
        args.update(kw)
        assert ssd.ssd_plan(_p(**args))["fused"] == 0, kw
    # fp32 otherwise: 64 columns per state-pass workgroup, chains split into groups up to four
    # workgroups per CU at 64-token chunks (here one chunk per group), then the scan
    f = ssd.ssd_plan(_p(seqlen=576, nheads=4, dstate=64, chunk=64, dtype="fp32"))
    assert (f["sp_group_chunks"], f["sp_groups"], f["sp_columns"], f["sp_workgroups"], f["scan"],
            f["co_head_blocked"], f["fused"]) == (1, 9, 64, 36, 1, 0, 0)
    f2 = ssd.ssd_plan(_p(seqlen=16384, nheads=32, dstate=256, chunk=256, dtype="fp32"))
    assert (f2["sp_group_chunks"], f2["sp_groups"], f2["sp_workgroups"]) == (32, 2, 256)
    # fp32 chunk output: two waves (one row tile each) for 64-token chunks below 1024
    # workgroups, else Q threads (Q/64 waves with two row tiles each)
    assert (f["co_workgroups"], f["co_threads"]) == (36, 128)
    f3 = ssd.ssd_plan(_p(batch=2, seqlen=4096, nheads=16, dstate=128, chunk=64, dtype="fp32"))
    assert (f3["co_workgroups"], f3["co_threads"]) == (2048, 64)
    assert ssd.ssd_plan(_p(batch=2, seqlen=4096, nheads=7, dstate=128, chunk=64, dtype="fp32"))["co_threads"] == 128
    assert f2["co_threads"] == 256
    # the plan refuses what the forward refuses
    with pytest.raises(ssd.SsdError) as ei:
        ssd.ssd_plan(_p(dstate=96))
    assert ei.value.status == 3


@pytest.mark.parametrize("kw,status", [
    # per-batch extents of x and of B / C: below 2^30 elements
    (dict(seqlen=(1 << 30) // (32 * 64) - 1, nheads=32, dstate=64), 0),
    (dict(seqlen=(1 << 30) // (32 * 64), nheads=32, dstate=64), 3),
    (dict(seqlen=(1 << 30) // 512 - 1, nheads=1, dstate=512), 0),
    (dict(seqlen=(1 << 30) // 512, nheads=1, dstate=512), 3),
    # batch * heads
    (dict(batch=65535, nheads=1, seqlen=64, dstate=64, chunk=64), 0),
    (dict(batch=65536, nheads=1, seqlen=64, dstate=64, chunk=64), 3),
    (dict(batch=1 << 40, nheads=4), 3),             # no overflow in the product
    (dict(batch=4, nheads=1 << 40, ngroups=1), 3),
    # the one-head output kernel's workgroup count
    (dict(batch=9362, nheads=7, ngroups=7, seqlen=(1 << 21) + 192, dstate=64, chunk=64), 3),
    (dict(batch=9362, nheads=7, ngroups=7, seqlen=1 << 15, dstate=64, chunk=64), 0),
    # ... and its work-items (2 * chunk per workgroup), counted in 32 bits
    (dict(batch=8192, nheads=1, seqlen=256 * 1024, dstate=64, chunk=256), 3),
    (dict(batch=8192, nheads=1, seqlen=256 * 1023, dstate=64, chunk=256), 0),
])
def test_validate_size_limits(kw, status):
    assert ssd.ssd_validate(_p(**kw)) == status


PLAN_SHAPES = [
    dict(),                                                     # headline
    dict(seqlen=65536, dstate=512, chunk=128),
    dict(batch=2, seqlen=2048, nheads=24, dstate=128),
    dict(seqlen=262144, nheads=16, ngroups=2, dstate=128),
    dict(seqlen=700, nheads=4, ngroups=2, dstate=384, chunk=128),
    dict(seqlen=300, nheads=3, dstate=64, chunk=64),
    dict(seqlen=256, nheads=4, dstate=64, chunk=64, dtype="fp32"),
    dict(seqlen=1, nheads=2, dstate=512, chunk=256),
]


@pytest.mark.parametrize("kw", PLAN_SHAPES)
def test_plan_candidates(kw):
    """The search space of the launch configuration (host only): ssd_plan's choice first,
    no duplicates, every candidate valid with a workspace size, the documented choices."""
    p = _p(**kw)
    cands = ssd.plan_candidates(p)
    assert cands[0] == ssd.ssd_plan(p)
    keys = [tuple(sorted(c.items())) for c in cands]
    assert len(set(keys)) == len(keys)
    nc = p.nchunks
    fused = [c for c in cands if c["fused"]]
    if fused:   # the one-launch forward: one workgroup of 256 threads per (batch, head, chunk
        # or final state, half of the headdim)
        assert len(fused) == 1 and fused[0] == ssd.ssd_plan(p)
        assert (fused[0]["co_workgroups"], fused[0]["co_threads"], fused[0]["sp_workgroups"]) == (
            2 * (nc + 1) * p.batch * p.nheads, 256, 0)
        assert ssd.ssd_workspace_bytes_planned(p, fused[0]) > 0
        cands = [c for c in cands if not c["fused"]]
    for c in cands:
        assert ssd.ssd_workspace_bytes_planned(p, c) > 0
        K, ng = c["sp_group_chunks"], c["sp_groups"]
        assert 1 <= K <= nc and ng == -(-nc // K) and c["scan"] == (ng > 1)
        assert p.dstate % c["sp_columns"] == 0
        assert c["sp_workgroups"] == p.batch * p.nheads * (p.dstate // c["sp_columns"]) * ng
        if c["sp_register_transposed"]:
            assert c["sp_columns"] == 256 and c["sp_threads"] == 256
        if c["co_head_blocked"]:
            assert (p.nheads // p.ngroups) % c["co_heads_per_block"] == 0
        else:
            assert c["co_heads_per_block"] == 1 and c["co_workgroups"] == nc * p.batch * p.nheads
    # the groupings: 1, 2, 3, 4, 6, 8, ... groups as far as the chain has chunks
    groups = {c["sp_groups"] for c in cands}
    for g in (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128):
        if g <= nc:
            assert -(-nc // -(-nc // g)) in groups
    if p.dtype == binding.SSD_F32:
        assert {(c["sp_columns"], c["sp_register_transposed"], c["co_head_blocked"]) for c in cands} == {(64, 0, 0)}
    else:
        kinds = {(c["sp_columns"], c["sp_register_transposed"]) for c in cands}
        want = {(cols, 0) for cols in (64, 128, 256) if p.dstate % cols == 0}
        want |= {(256, 1)} if p.dstate % 256 == 0 else set()
        assert kinds == want
    # the workspace follows the grouping
    one = [c for c in cands if c["sp_groups"] == 1]
    assert one and ssd.ssd_workspace_bytes_planned(p, one[0]) <= min(
        ssd.ssd_workspace_bytes_planned(p, c) for c in cands)


def test_plan_candidates_capacity():
    lib = binding.lib()
    p = _p()
    count = ctypes.c_int32(-1)
    assert lib.ssd_plan_candidates(ctypes.byref(p), None, 0, ctypes.byref(count)) == 0
    n = count.value
    assert n > 10
    arr = (binding.SsdLaunchPlan * 3)()
    assert lib.ssd_plan_candidates(ctypes.byref(p), arr, 3, ctypes.byref(count)) == 0
    assert count.value == n
    assert {f: getattr(arr[0], f) for f, _ in binding.SsdLaunchPlan._fields_} == ssd.ssd_plan(p)
    assert lib.ssd_plan_candidates(ctypes.byref(p), None, 3, ctypes.byref(count)) == 1
    assert lib.ssd_plan_candidates(ctypes.byref(p), arr, -1, ctypes.byref(count)) == 1
    assert lib.ssd_plan_candidates(ctypes.byref(p), arr, 3, None) == 1
    assert lib.ssd_plan_candidates(ctypes.byref(_p(dstate=96)), arr, 3, ctypes.byref(count)) == 3


def _altered(plan, **kw):
    q = dict(plan)
    q.update(kw)
    return q


def test_invalid_plans_rejected_without_launching():
    """A plan the kernels cannot run is refused with SSD_ERR_PLAN before any launch, and
    has no workspace size (host only: fake device pointers are never touched)."""
    lib = binding.lib()
    p = _p()
    d = ssd.ssd_plan(p)
    bad = [
        _altered(d, sp_columns=96),
        _altered(d, sp_columns=512),
        _altered(d, sp_register_transposed=1, sp_columns=128, sp_workgroups=d["sp_workgroups"] * 2),
        _altered(d, sp_group_chunks=0),
        _altered(d, sp_group_chunks=65),
        _altered(d, sp_groups=7),                      # not ceil(nc / K)
        _altered(d, sp_workgroups=d["sp_workgroups"] + 1),
        _altered(d, co_heads_per_block=3),             # does not divide the heads per group
        _altered(d, co_threads=256),
        _altered(d, scan=0),
        _altered(d, co_head_blocked=2),
    ]
    fake = ctypes.c_void_p(256)
    for q in bad:
        assert ssd.ssd_workspace_bytes_planned(p, q) == 0, q
        st = lib.ssd_forward_planned(ctypes.byref(p), ctypes.byref(binding._plan_struct(q)),
                                     *([fake] * 6), None, fake, None, fake, 10**12, 0, 3, None, None)
        assert st == 8, q
    # the one-head kernel for 64-token chunks only; fp32 takes no other state-pass kernel
    p64 = _p(chunk=64)
    d64 = ssd.ssd_plan(p64)
    assert ssd.ssd_workspace_bytes_planned(p64, _altered(d64, co_head_blocked=1)) == 0
    pf = _p(dtype="fp32", dstate=128, chunk=64)
    df = ssd.ssd_plan(pf)
    assert ssd.ssd_workspace_bytes_planned(pf, _altered(df, sp_columns=128,
                                                        sp_workgroups=df["sp_workgroups"] // 2)) == 0
    # a valid plan other than the default, and the NULL plan, pass the checks and stop at
    # the next one (workspace too small)
    other = [c for c in ssd.plan_candidates(p) if c != d][0]
    for q in (ctypes.byref(binding._plan_struct(other)), None):
        assert lib.ssd_forward_planned(ctypes.byref(p), q, *([fake] * 6), None, fake, None, fake,
                                       100, 0, 3, None, None) == 4
    # stage range
    for first, last in ((-1, 3), (0, 4), (3, 2)):
        assert lib.ssd_forward_planned(ctypes.byref(p), None, *([fake] * 6), None, fake, None,
                                       fake, 10**12, first, last, None, None) == 3
    assert lib.ssd_last_hip_error() == 0
