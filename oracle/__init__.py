"""fp64 CPU oracle for the Mamba-2 SSD chunked forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and does not import it.

The arithmetic lives in ``ssd_oracle.c`` (built with gcc -O2, no fast-math):

* :func:`forward` runs the per-token recurrence of "基于 NVIDIA CUDA Tile 加速
  Mamba-2 高性能前向传播内核" (dbyun.net), section "Mamba-2 架构":
  ``h_t = exp(A dt_t) h_{t-1} + dt_t x_t (outer) B_t``, ``y_t = h_t . C_t + D x_t``,
  in double precision, one (batch, head) pair at a time, optionally recording the
  state at every chunk start (what the "fwd_pass_state" kernel stores).
* :func:`chunk_cumsum` is the definition of the first kernel's output (section
  "Kernel 1：计算累积和"): the within-chunk inclusive sum of ``A[h] * dt``
  times log2(e).

Inputs may be numpy arrays (float64 / float32) or torch CPU tensors (float64,
float32 or bfloat16); bf16 values are widened exactly, so the oracle sees the
very values the GPU reads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ssd_oracle.c")
# SSD_ORACLE_LIBRARY points the pins at another build of the oracle (the planted-mistake
# test builds deliberately wrong copies of ssd_oracle.c and checks that the pins fail)
LIBRARY = os.environ.get("SSD_ORACLE_LIBRARY") or os.path.join(_HERE, "libssd_oracle.so")

_F64, _F32, _BF16 = 0, 1, 2
_lib = None


def build(force: bool = True) -> str:
    """Compile ssd_oracle.c into libssd_oracle.so with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(LIBRARY):
        compile_oracle(SOURCE, LIBRARY)
    return LIBRARY


def compile_oracle(source: str, library: str) -> None:
    """gcc -O2 (no fast-math) of an oracle source file into a shared library."""
    tmp = library + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-shared", "-fPIC",
                           "-pthread", source, "-o", tmp, "-lm"])
    os.replace(tmp, library)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            build(force=False)
        lib = ctypes.CDLL(LIBRARY)
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
        lib.ssd_oracle_forward.restype = ctypes.c_int
        lib.ssd_oracle_forward.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                           vp, vp, vp, vp, dp, dp, dp, vp, i64, i64,
                                           dp, dp, dp, ctypes.c_int]
        lib.ssd_oracle_chunk_cumsum.restype = ctypes.c_int
        lib.ssd_oracle_chunk_cumsum.argtypes = [i64, i64, i64, ctypes.c_int, vp, dp, i64, dp, dp]
        _lib = lib
    return _lib


def _storage(a):
    """Return (contiguous numpy array, dtype code) holding exactly the stored values."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                return a.view(torch.int16).numpy().view(np.uint16), _BF16
            a = a.numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    a = np.ascontiguousarray(a)
    if a.dtype == np.float64:
        return a, _F64
    if a.dtype == np.float32:
        return a, _F32
    raise TypeError(f"oracle input dtype {a.dtype} not supported (float64, float32, bfloat16)")


def _f64(a):
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def forward(x, dt, A, B, C, D, h0=None, *, units=None, chunk: int = 0, want_y: bool = True,
            want_hT: bool = True, nthreads: int | None = None):
    """Sequential fp64 recurrence.

    Shapes: x [b,L,H,P], dt [b,L,H], B and C [b,L,G,N], A and D [H], h0 [b,H,P,N] or None.
    ``units``: iterable of flat (b*H + h) ids to compute (default: all, in order).
    Returns a dict with ``units`` and, as requested, ``y`` [n,L,P], ``hT`` [n,P,N] and
    ``snaps`` [n, ceil(L/chunk), P, N] (the state at each chunk start; ``chunk`` > 0).
    """
    xs, code = _storage(x)
    dts, c2 = _storage(dt)
    Bs, c3 = _storage(B)
    Cs, c4 = _storage(C)
    if len({code, c2, c3, c4}) != 1:
        raise TypeError("x, dt, B and C must share one storage dtype")
    b, L, H, P = xs.shape
    G, N = Bs.shape[2], Bs.shape[3]
    if dts.shape != (b, L, H) or Bs.shape != (b, L, G, N) or Cs.shape != (b, L, G, N):
        raise ValueError("inconsistent input shapes")
    A64, D64, h064 = _f64(A), _f64(D), _f64(h0)
    if A64.shape != (H,) or D64.shape != (H,):
        raise ValueError("A and D must have shape [H]")
    if h064 is not None and h064.shape != (b, H, P, N):
        raise ValueError("h0 must have shape [b,H,P,N]")
    if units is None:
        u = np.arange(b * H, dtype=np.int64)
    else:
        u = np.ascontiguousarray(np.asarray(list(units), dtype=np.int64))
    n = len(u)
    y = np.empty((n, L, P), np.float64) if want_y else None
    hT = np.empty((n, P, N), np.float64) if want_hT else None
    snaps = None
    if chunk > 0:
        nc = -(-L // chunk)
        snaps = np.empty((n, nc, P, N), np.float64)
    rc = _load().ssd_oracle_forward(b, L, H, G, P, N, code, _ptr(xs), _ptr(dts), _ptr(Bs),
                                    _ptr(Cs), _ptr(A64), _ptr(D64), _ptr(h064), _ptr(u), n,
                                    int(chunk), _ptr(y), _ptr(hT), _ptr(snaps),
                                    int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"ssd_oracle_forward rejected its arguments (code {rc})")
    return {"units": u, "y": y, "hT": hT, "snaps": snaps}


def forward_full(x, dt, A, B, C, D, h0=None, *, chunk: int = 0, nthreads: int | None = None):
    """All units; returns y [b,L,H,P], hT [b,H,P,N] and snaps [b,H,nc,P,N] (if chunk > 0)."""
    out = forward(x, dt, A, B, C, D, h0, chunk=chunk, nthreads=nthreads)
    b, L, H, P = tuple(x.shape)
    N = tuple(B.shape)[3]
    res = {
        "y": out["y"].reshape(b, H, L, P).transpose(0, 2, 1, 3).copy(),
        "hT": out["hT"].reshape(b, H, P, N),
    }
    if out["snaps"] is not None:
        res["snaps"] = out["snaps"].reshape(b, H, -1, P, N)
    return res


def chunk_cumsum(dt, A, chunk: int):
    """G2 [b,H,L] = log2(e) * within-chunk inclusive cumsum of A[h]*dt; also dt as [b,H,L] fp64."""
    dts, code = _storage(dt)
    b, L, H = dts.shape
    A64 = _f64(A)
    G2 = np.empty((b, H, L), np.float64)
    dtc = np.empty((b, H, L), np.float64)
    rc = _load().ssd_oracle_chunk_cumsum(b, L, H, code, _ptr(dts), _ptr(A64), int(chunk),
                                         _ptr(G2), _ptr(dtc))
    if rc != 0:
        raise ValueError(f"ssd_oracle_chunk_cumsum rejected its arguments (code {rc})")
    return G2, dtc
