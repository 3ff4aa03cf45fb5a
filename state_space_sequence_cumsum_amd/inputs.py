"""Seeded synthetic inputs for the SSD forward pass.

This module draws random inputs and nothing else: it holds none of the
method's arithmetic, and both the GPU path and the CPU oracle are fed from it.

Recipe (fixed draw order A, D, dt, x, B, C, h0 from one CPU ``torch.Generator``):

* ``A[h] = -exp(U(log 1, log 16))``           per-head decay rate, in [-16, -1]
* ``D[h] ~ U(0, 1)``                          per-head skip weight
* ``dt = softplus(N(0,1) + dt_shift)``        per (token, head), dt_shift = -4 (or -6)
* ``x, B, C ~ N(0, 1)``
* ``h0 = 0.1 * N(0, 1)``                      only where the workload has an initial state

Values are drawn in fp32; for bf16 workloads x, dt, B and C are then rounded to
bf16 (round-to-nearest-even, torch's ``.to(torch.bfloat16)``).  A, D and h0 stay fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "fp32" or "bf16": storage type of x, dt, B, C and y
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dt_shift: float = -4.0
    has_h0: bool = False

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the study, smallest first, then the pages' own usage
# example.  The 16K-token, N=256 one is the headline throughput case.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("fp32_b1_L256_H4_P64_N64_Q64", "fp32", 1, 256, 4, 64, 64, 1, 64),
        Workload("bf16_b2_L2048_H24_P64_N128_Q256", "bf16", 2, 2048, 24, 64, 128, 1, 256),
        Workload("bf16_b1_L16384_H32_P64_N256_Q256", "bf16", 1, 16384, 32, 64, 256, 1, 256,
                 has_h0=True),
        Workload("bf16_b1_L65536_H32_P64_N512_Q128", "bf16", 1, 65536, 32, 64, 512, 1, 128),
        Workload("bf16_b1_L262144_H16_G2_P64_N128_Q256", "bf16", 1, 262144, 16, 64, 128, 2, 256,
                 dt_shift=-6.0, has_h0=True),
        # the usage example of the dbyun.net page (section "Mamba-2 前向传播性能基准测试"):
        # batch 4, 16K tokens, 8 heads, one group, state 128, head 64, chunk 128, bf16
        # inputs with an fp32 state; the example passes no initial state
        Workload("bf16_b4_L16384_H8_P64_N128_Q128", "bf16", 4, 16384, 8, 64, 128, 1, 128),
    ]
}
HEADLINE = "bf16_b1_L16384_H32_P64_N256_Q256"
SMALL = "fp32_b1_L256_H4_P64_N64_Q64"


def torch_dtype(name: str) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(w: Workload, seed: int = 0, device="cpu") -> dict:
    """Draw one set of inputs for workload ``w``.

    Returns torch tensors on ``device``: x [b,L,H,P], dt [b,L,H], A [H], B and C
    [b,L,G,N], D [H], and h0 [b,H,P,N] or None.  The generator lives on ``device``:
    every parity input is drawn on the CPU; a GPU draw (same laws, other values)
    only feeds timing runs too large to draw on the host quickly.
    """
    g = torch.Generator(device=device).manual_seed(int(seed))
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    kw = {"generator": g, "device": device}
    A = -torch.exp(torch.empty(H, device=device).uniform_(math.log(1.0), math.log(16.0),
                                                          generator=g))
    D = torch.empty(H, device=device).uniform_(0.0, 1.0, generator=g)
    dt = torch.nn.functional.softplus(torch.randn(b, L, H, **kw) + w.dt_shift)
    x = torch.randn(b, L, H, P, **kw)
    B = torch.randn(b, L, G, N, **kw)
    C = torch.randn(b, L, G, N, **kw)
    h0 = 0.1 * torch.randn(b, H, P, N, **kw) if w.has_h0 else None
    td = torch_dtype(w.dtype)
    return {
        "x": x.to(td).contiguous(),
        "dt": dt.to(td).contiguous(),
        "A": A.contiguous(),
        "B": B.to(td).contiguous(),
        "C": C.to(td).contiguous(),
        "D": D.contiguous(),
        "h0": None if h0 is None else h0.contiguous(),
    }
