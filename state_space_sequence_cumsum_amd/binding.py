"""ctypes binding of libssd (include/ssd.h).

Argument marshalling only: every function checks tensor placement, dtype, shape
and contiguity, turns tensors into device pointers and calls the C entry point
of the same name on the current (or given) HIP stream.  Outputs that the caller
does not pass are allocated with ``torch.empty`` on the inputs' device.  There is
no CPU or PyTorch fallback: when libssd.so is missing or a call fails, this
module raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libssd.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "ssd.h")

SSD_F32, SSD_BF16 = 0, 1
FORWARD_EVENTS = 5      # SSD_FORWARD_EVENTS: marks around stage 1, state pass, group scan, stage 3
STATUS = {0: "SSD_OK", 1: "SSD_ERR_NULL_ARG", 2: "SSD_ERR_BAD_SHAPE", 3: "SSD_ERR_UNSUPPORTED",
          4: "SSD_ERR_WORKSPACE", 5: "SSD_ERR_HIP", 6: "SSD_ERR_MISALIGNED", 7: "SSD_ERR_SCRATCH",
          8: "SSD_ERR_PLAN"}
SCRATCH_BYTES = 128 << 20   # SSD_SCRATCH_BYTES: the static workspace of ssd_forward_noalloc


class SsdError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str = ""):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({detail})")


class SsdProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("ngroups", ctypes.c_int64), ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("dtype", ctypes.c_int32)]

    def __repr__(self):
        return ("SsdProblem(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")")

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk)


class SsdLaunchPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "sp_group_chunks", "sp_groups", "sp_columns", "sp_workgroups", "scan", "co_head_blocked",
        "co_heads_per_block", "co_column_split", "co_workgroups", "co_threads",
        "sp_register_transposed", "sp_threads", "fused")]


_lib = None


def lib():
    """Load libssd.so (built in-tree by build.py); raise if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is missing: build it first (python -m "
                               "state_space_sequence_cumsum_amd.build or __graft_entry__.build())")
        L = ctypes.CDLL(LIBRARY)
        P, vp, st = ctypes.POINTER(SsdProblem), ctypes.c_void_p, ctypes.c_int
        L.ssd_validate.argtypes, L.ssd_validate.restype = [P], st
        L.ssd_workspace_bytes.argtypes, L.ssd_workspace_bytes.restype = [P], ctypes.c_size_t
        L.ssd_workspace_layout.argtypes = [P] + [ctypes.POINTER(ctypes.c_size_t)] * 3
        L.ssd_workspace_layout.restype = st
        L.ssd_chunk_cumsum.argtypes, L.ssd_chunk_cumsum.restype = [P, vp, vp, vp, vp, vp], st
        L.ssd_state_pass.argtypes, L.ssd_state_pass.restype = [P, vp, vp, vp, vp, vp, vp, vp, vp], st
        L.ssd_chunk_out.argtypes, L.ssd_chunk_out.restype = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp], st
        L.ssd_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.ssd_forward.restype = st
        L.ssd_forward_timed.argtypes = L.ssd_forward.argtypes + [ctypes.POINTER(vp)]
        L.ssd_forward_timed.restype = st
        L.ssd_forward_stage.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        ctypes.c_size_t, ctypes.c_int, vp]
        L.ssd_forward_stage.restype = st
        L.ssd_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.ssd_forward_noalloc.restype = st
        L.ssd_step.argtypes, L.ssd_step.restype = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp], st
        L.ssd_plan.argtypes, L.ssd_plan.restype = [P, ctypes.POINTER(SsdLaunchPlan)], st
        L.ssd_plan_candidates.argtypes = [P, ctypes.POINTER(SsdLaunchPlan), ctypes.c_int32,
                                          ctypes.POINTER(ctypes.c_int32)]
        L.ssd_plan_candidates.restype = st
        L.ssd_workspace_bytes_planned.argtypes = [P, ctypes.POINTER(SsdLaunchPlan)]
        L.ssd_workspace_bytes_planned.restype = ctypes.c_size_t
        L.ssd_forward_planned.argtypes = [P, ctypes.POINTER(SsdLaunchPlan), vp, vp, vp, vp, vp, vp,
                                          vp, vp, vp, vp, ctypes.c_size_t, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.POINTER(vp), vp]
        L.ssd_forward_planned.restype = st
        L.ssd_status_string.argtypes, L.ssd_status_string.restype = [st], ctypes.c_char_p
        L.ssd_last_hip_error.argtypes, L.ssd_last_hip_error.restype = [], ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/ssd.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_0-9]+)\s*\(", text)))


def _raise(status: int, what: str):
    if status != 0:
        L = lib()
        detail = L.ssd_status_string(status).decode()
        if status == 5:
            detail += f"; hipError_t {L.ssd_last_hip_error()}"
        raise SsdError(status, what, detail)


# ---------------------------------------------------------------------------
# problem descriptors (host only)
# ---------------------------------------------------------------------------
def make_problem(batch, seqlen, nheads, ngroups, headdim, dstate, chunk, dtype) -> SsdProblem:
    code = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16, "fp32": SSD_F32, "bf16": SSD_BF16}
    return SsdProblem(int(batch), int(seqlen), int(nheads), int(ngroups), int(headdim), int(dstate),
                      int(chunk), code.get(dtype, dtype) if not isinstance(dtype, int) else dtype)


def problem_of(x: torch.Tensor, B: torch.Tensor, chunk: int) -> SsdProblem:
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return make_problem(b, L, H, G, P, N, chunk, x.dtype)


def ssd_validate(problem: SsdProblem) -> int:
    return lib().ssd_validate(ctypes.byref(problem))


def ssd_workspace_bytes(problem: SsdProblem) -> int:
    return lib().ssd_workspace_bytes(ctypes.byref(problem))


def ssd_workspace_layout(problem: SsdProblem) -> tuple[int, int, int]:
    """Byte offsets of (G2, dtT, S) inside an ssd_forward workspace."""
    offs = [ctypes.c_size_t() for _ in range(3)]
    _raise(lib().ssd_workspace_layout(ctypes.byref(problem), *[ctypes.byref(o) for o in offs]),
           "ssd_workspace_layout")
    return tuple(o.value for o in offs)


def ssd_plan(problem: SsdProblem) -> dict:
    """How ssd_forward launches `problem` (host only): field name -> value."""
    plan = SsdLaunchPlan()
    _raise(lib().ssd_plan(ctypes.byref(problem), ctypes.byref(plan)), "ssd_plan")
    return {n: getattr(plan, n) for n, _ in SsdLaunchPlan._fields_}


def _plan_struct(plan) -> SsdLaunchPlan:
    """An SsdLaunchPlan from a field-name dict (as ssd_plan / plan_candidates return) or
    an SsdLaunchPlan."""
    if isinstance(plan, SsdLaunchPlan):
        return plan
    missing = [n for n, _ in SsdLaunchPlan._fields_ if n not in plan]
    if missing:
        raise ValueError(f"launch plan lacks fields {missing}")
    return SsdLaunchPlan(**{n: int(plan[n]) for n, _ in SsdLaunchPlan._fields_})


def plan_candidates(problem: SsdProblem) -> list[dict]:
    """The forward's launch configurations for `problem` (host only; ssd_plan_candidates):
    a list of field-name dicts, ssd_plan's choice first."""
    count = ctypes.c_int32(0)
    _raise(lib().ssd_plan_candidates(ctypes.byref(problem), None, 0, ctypes.byref(count)),
           "ssd_plan_candidates")
    arr = (SsdLaunchPlan * max(1, count.value))()
    _raise(lib().ssd_plan_candidates(ctypes.byref(problem), arr, count.value, ctypes.byref(count)),
           "ssd_plan_candidates")
    return [{n: getattr(arr[i], n) for n, _ in SsdLaunchPlan._fields_} for i in range(count.value)]


def ssd_workspace_bytes_planned(problem: SsdProblem, launch_plan=None) -> int:
    """Workspace bytes of the forward under `launch_plan` (None: ssd_plan's); 0 when the
    problem or the plan is not valid."""
    plan = None if launch_plan is None else ctypes.byref(_plan_struct(launch_plan))
    return lib().ssd_workspace_bytes_planned(ctypes.byref(problem), plan)


def ssd_status_string(status: int) -> str:
    return lib().ssd_status_string(status).decode()


# ---------------------------------------------------------------------------
# device entry points
# ---------------------------------------------------------------------------
def _dev(t, name, dtype, shape, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, device):
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dims(p: SsdProblem):
    return p.batch, p.seqlen, p.nheads, p.ngroups, p.headdim, p.dstate, p.chunk, p.nchunks


def _io_dtype(p: SsdProblem):
    return torch.bfloat16 if p.dtype == SSD_BF16 else torch.float32


def ssd_chunk_cumsum(problem: SsdProblem, dt, A, G2=None, dtT=None, stream=None):
    """Stage 1.  Returns (G2, dtT), both float32 [b, H, nc*Q]."""
    b, L, H, G, P, N, Q, nc = _dims(problem)
    dev = dt.device
    _dev(dt, "dt", _io_dtype(problem), (b, L, H), None)
    _dev(A, "A", torch.float32, (H,), dev)
    out = []
    for name, t in (("G2", G2), ("dtT", dtT)):
        if t is None:
            t = torch.empty(b, H, nc * Q, device=dev, dtype=torch.float32)
        out.append(_dev(t, name, torch.float32, (b, H, nc * Q), dev))
    G2, dtT = out
    _raise(lib().ssd_chunk_cumsum(ctypes.byref(problem), _ptr(dt), _ptr(A), _ptr(G2), _ptr(dtT),
                                  _stream(stream, dev)), "ssd_chunk_cumsum")
    return G2, dtT


def ssd_state_pass(problem: SsdProblem, x, B, G2, dtT, h0=None, S=None, hT=None, want_final=True,
                   stream=None):
    """Stage 2.  Returns (S [b,H,nc,P,N] in the input dtype, hT [b,H,P,N] float32 or None)."""
    b, L, H, G, P, N, Q, nc = _dims(problem)
    io = _io_dtype(problem)
    dev = x.device
    _dev(x, "x", io, (b, L, H, P), None)
    _dev(B, "B", io, (b, L, G, N), dev)
    _dev(G2, "G2", torch.float32, (b, H, nc * Q), dev)
    _dev(dtT, "dtT", torch.float32, (b, H, nc * Q), dev)
    _dev(h0, "h0", torch.float32, (b, H, P, N), dev)
    if S is None:
        S = torch.empty(b, H, nc, P, N, device=dev, dtype=io)
    if hT is None and want_final:
        hT = torch.empty(b, H, P, N, device=dev, dtype=torch.float32)
    _dev(S, "S", io, (b, H, nc, P, N), dev)
    _dev(hT, "hT", torch.float32, (b, H, P, N), dev)
    _raise(lib().ssd_state_pass(ctypes.byref(problem), _ptr(x), _ptr(B), _ptr(G2), _ptr(dtT),
                                _ptr(h0), _ptr(S), _ptr(hT), _stream(stream, dev)), "ssd_state_pass")
    return S, hT


def ssd_chunk_out(problem: SsdProblem, x, B, C, G2, dtT, S, D, y=None, stream=None):
    """Stage 3.  Returns y [b, L, H, P] in the input dtype."""
    b, L, H, G, P, N, Q, nc = _dims(problem)
    io = _io_dtype(problem)
    dev = x.device
    _dev(x, "x", io, (b, L, H, P), None)
    _dev(B, "B", io, (b, L, G, N), dev)
    _dev(C, "C", io, (b, L, G, N), dev)
    _dev(G2, "G2", torch.float32, (b, H, nc * Q), dev)
    _dev(dtT, "dtT", torch.float32, (b, H, nc * Q), dev)
    _dev(S, "S", io, (b, H, nc, P, N), dev)
    _dev(D, "D", torch.float32, (H,), dev)
    if y is None:
        y = torch.empty(b, L, H, P, device=dev, dtype=io)
    _dev(y, "y", io, (b, L, H, P), dev)
    _raise(lib().ssd_chunk_out(ctypes.byref(problem), _ptr(x), _ptr(B), _ptr(C), _ptr(G2),
                               _ptr(dtT), _ptr(S), _ptr(D), _ptr(y), _stream(stream, dev)),
           "ssd_chunk_out")
    return y


def workspace_for(problem: SsdProblem, device, launch_plan=None) -> torch.Tensor:
    n = ssd_workspace_bytes_planned(problem, launch_plan)
    if n == 0:
        _raise(ssd_validate(problem) or 8, "ssd_workspace_bytes_planned")
    return torch.empty(n, device=device, dtype=torch.uint8)


def _io_args(x, dt, A, B, C, D, h0, chunk, y, hT, want_final):
    """Checked problem, inputs and outputs of a forward call (outputs allocated here
    when not given)."""
    problem = problem_of(x, B, chunk)
    b, L, H, G, P, N, Q, nc = _dims(problem)
    io = _io_dtype(problem)
    dev = x.device
    _dev(x, "x", io, (b, L, H, P), None)
    _dev(dt, "dt", io, (b, L, H), dev)
    _dev(A, "A", torch.float32, (H,), dev)
    _dev(B, "B", io, (b, L, G, N), dev)
    _dev(C, "C", io, (b, L, G, N), dev)
    _dev(D, "D", torch.float32, (H,), dev)
    _dev(h0, "h0", torch.float32, (b, H, P, N), dev)
    if y is None:
        y = torch.empty(b, L, H, P, device=dev, dtype=io)
    if hT is None and want_final:
        hT = torch.empty(b, H, P, N, device=dev, dtype=torch.float32)
    _dev(y, "y", io, (b, L, H, P), dev)
    _dev(hT, "hT", torch.float32, (b, H, P, N), dev)
    return problem, dev, y, hT


def _forward_args(x, dt, A, B, C, D, h0, chunk, y, hT, want_final, workspace, stream,
                  launch_plan=None):
    """Checked ctypes arguments of ssd_forward, with the outputs and the workspace
    (allocated here when not given, sized for `launch_plan`)."""
    problem, dev, y, hT = _io_args(x, dt, A, B, C, D, h0, chunk, y, hT, want_final)
    if workspace is None:
        workspace = workspace_for(problem, dev, launch_plan)
    if not workspace.is_cuda or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    nbytes = workspace.numel() * workspace.element_size()
    args = (ctypes.byref(problem), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            _ptr(h0), _ptr(y), _ptr(hT), _ptr(workspace), nbytes, _stream(stream, dev))
    return problem, args, y, hT, workspace


def _event_array(events):
    if len(events) != FORWARD_EVENTS or not all(getattr(e, "cuda_event", 0) for e in events):
        raise ValueError(f"events must be {FORWARD_EVENTS} torch.cuda.Event objects "
                         "recorded at least once")
    return (ctypes.c_void_p * FORWARD_EVENTS)(*[e.cuda_event for e in events])


def _planned(args, plan, first, last, events):
    """ssd_forward_planned with the ssd_forward argument tuple `args`."""
    return lib().ssd_forward_planned(args[0], plan, *args[1:-1], int(first), int(last), events,
                                     args[-1])


def ssd_forward(x, dt, A, B, C, D, h0=None, *, chunk: int, y=None, hT=None, want_final=True,
                workspace=None, stream=None, events=None, launch_plan=None):
    """Whole forward pass.  Returns (y [b,L,H,P], hT [b,H,P,N] float32 or None).

    ``events``: optional ``FORWARD_EVENTS`` (5) recorded-once ``torch.cuda.Event``
    objects; they are re-recorded on the launch stream around each of the four
    launches (stage 1, state pass, group scan, stage 3; ssd_forward_timed).
    ``launch_plan``: a candidate of ``plan_candidates`` to run instead of ssd_plan's
    choice (ssd_forward_planned); the workspace must then be sized for it.
    """
    _, args, y, hT, _ = _forward_args(x, dt, A, B, C, D, h0, chunk, y, hT, want_final, workspace,
                                      stream, launch_plan)
    if launch_plan is not None:
        arr = None if events is None else _event_array(events)
        _raise(_planned(args, ctypes.byref(_plan_struct(launch_plan)), 0, FORWARD_EVENTS - 2, arr),
               "ssd_forward_planned")
    elif events is None:
        _raise(lib().ssd_forward(*args), "ssd_forward")
    else:
        _raise(lib().ssd_forward_timed(*args, _event_array(events)), "ssd_forward_timed")
    return y, hT


def ssd_forward_noalloc(x, dt, A, B, C, D, h0=None, *, chunk: int, y=None, hT=None,
                        want_final=True, stream=None):
    """ssd_forward with the library's static device scratch as the workspace: the C call
    allocates nothing (pass y, and hT unless want_final is False, to keep this wrapper
    from allocating them).  Returns (y, hT).  Raises SsdError with SSD_ERR_SCRATCH when
    the problem needs more than SCRATCH_BYTES of workspace."""
    problem, dev, y, hT = _io_args(x, dt, A, B, C, D, h0, chunk, y, hT, want_final)
    _raise(lib().ssd_forward_noalloc(ctypes.byref(problem), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                     _ptr(C), _ptr(D), _ptr(h0), _ptr(y), _ptr(hT),
                                     _stream(stream, dev)), "ssd_forward_noalloc")
    return y, hT


class ForwardPlan:
    """ssd_forward bound to fixed tensors: the arguments are checked and the outputs and
    workspace allocated once, and run() only calls the C entry point (the caller refills
    the inputs in place between calls).  The plan keeps its tensors alive; the stream is
    fixed when the plan is made (default: the current stream), so a plan made for a
    capture stream can be recorded into a HIP graph (the forward allocates, clears and
    synchronises nothing)."""

    def __init__(self, x, dt, A, B, C, D, h0=None, *, chunk: int, y=None, hT=None,
                 want_final=True, workspace=None, stream=None, launch_plan=None):
        self._keep = (x, dt, A, B, C, D, h0)
        self._problem, self._args, self.y, self.hT, self.workspace = _forward_args(
            x, dt, A, B, C, D, h0, chunk, y, hT, want_final, workspace, stream, launch_plan)
        # the launch configuration: ssd_plan's choice (plain ssd_forward) or the caller's
        self.launch_plan = (ssd_plan(self._problem) if launch_plan is None
                            else {n: getattr(_plan_struct(launch_plan), n)
                                  for n, _ in SsdLaunchPlan._fields_})
        self._plan = None if launch_plan is None else _plan_struct(launch_plan)
        self._fn = lib().ssd_forward

    def run(self):
        """One forward; returns (y, hT) (the same tensors every call)."""
        if self._plan is None:
            st = self._fn(*self._args)
        else:
            st = _planned(self._args, ctypes.byref(self._plan), 0, FORWARD_EVENTS - 2, None)
        if st != 0:
            _raise(st, "ssd_forward")
        return self.y, self.hT

    def run_stage(self, stage: int):
        """Launch one stage of the forward alone (0 chunk cumsum, 1 state pass, 2 group scan,
        3 chunk output; ssd_forward_stage, or ssd_forward_planned under a caller's plan) on
        the plan's workspace, for timing one kernel."""
        if self._plan is None:
            st = lib().ssd_forward_stage(*self._args[:-1], int(stage), self._args[-1])
        else:
            st = _planned(self._args, ctypes.byref(self._plan), stage, stage, None)
        if st != 0:
            _raise(st, "ssd_forward_stage")

    def run_timed(self, events):
        """One forward with FORWARD_EVENTS marks around its launches (see ssd_forward)."""
        arr = _event_array(events)
        if self._plan is None:
            st = lib().ssd_forward_timed(*self._args, arr)
        else:
            st = _planned(self._args, ctypes.byref(self._plan), 0, FORWARD_EVENTS - 2, arr)
        if st != 0:
            _raise(st, "ssd_forward_timed")
        return self.y, self.hT


def _step_args(x, dt, A, B, C, D, h, y, stream):
    """Checked ctypes arguments of ssd_step (and the output tensor y)."""
    if x.dim() != 3 or B.dim() != 3:
        raise ValueError("ssd_step takes x [b,H,P] and B [b,G,N]")
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    problem = make_problem(b, 1, H, G, P, N, 0, x.dtype)
    io = _io_dtype(problem)
    dev = x.device
    _dev(x, "x", io, (b, H, P), None)
    _dev(dt, "dt", io, (b, H), dev)
    _dev(A, "A", torch.float32, (H,), dev)
    _dev(B, "B", io, (b, G, N), dev)
    _dev(C, "C", io, (b, G, N), dev)
    _dev(D, "D", torch.float32, (H,), dev)
    _dev(h, "h", torch.float32, (b, H, P, N), dev)
    if y is None:
        y = torch.empty(b, H, P, device=dev, dtype=io)
    _dev(y, "y", io, (b, H, P), dev)
    args = (ctypes.byref(problem), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            _ptr(h), _ptr(y), _stream(stream, dev))
    return problem, args, y


def ssd_step(x, dt, A, B, C, D, h, *, y=None, stream=None):
    """One decode step.  x [b,H,P], dt [b,H], B and C [b,G,N] (input dtype), A and D [H]
    float32, h [b,H,P,N] float32 (updated in place).  Returns y [b,H,P]."""
    _, args, y = _step_args(x, dt, A, B, C, D, h, y, stream)
    _raise(lib().ssd_step(*args), "ssd_step")
    return y


class StepPlan:
    """ssd_step bound to fixed tensors, for decode loops: the arguments are checked once,
    and run() only calls the C entry point (the caller refills x, dt, B and C in place
    between calls; h is updated in place by each call).  The tensors are kept alive by
    the plan; the stream is fixed when the plan is made (default: the current stream)."""

    def __init__(self, x, dt, A, B, C, D, h, *, y=None, stream=None):
        self._keep = (x, dt, A, B, C, D, h)
        self._problem, self._args, self.y = _step_args(x, dt, A, B, C, D, h, y, stream)
        self._fn = lib().ssd_step

    def run(self):
        """One step; returns y (the same tensor every call)."""
        st = self._fn(*self._args)
        if st != 0:
            _raise(st, "ssd_step")
        return self.y


def workspace_views(problem: SsdProblem, workspace: torch.Tensor) -> dict:
    """Typed views (G2, dtT, S) of an ssd_forward workspace tensor."""
    b, L, H, G, P, N, Q, nc = _dims(problem)
    g2, dtt, so = ssd_workspace_layout(problem)
    cnt = b * H * nc * Q
    f32 = lambda off: workspace[off:off + 4 * cnt].view(torch.float32).view(b, H, nc * Q)
    io = _io_dtype(problem)
    es = 2 if io == torch.bfloat16 else 4
    S = workspace[so:so + es * b * H * nc * P * N].view(io).view(b, H, nc, P, N)
    return {"G2": f32(g2), "dtT": f32(dtt), "S": S}
