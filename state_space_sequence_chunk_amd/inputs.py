"""Seeded synthetic inputs for the SSD forward pass.

This module only draws random numbers and casts them; it contains none of the method's
arithmetic, so both the GPU path's tests and the CPU oracle may consume what it makes.

Workloads are shaped like Mamba-2 layers. Per-tensor distributions:

  x       ~ N(0, 1)                                   input dtype (bf16 or fp32)
  B, C    ~ N(0, 1) / sqrt(dstate)                    input dtype
  dt      = exp(U(ln 1e-3, ln 1e-1))  (log-uniform)   input dtype
  A[h]    = -exp(U(0, ln 16))        (in [-16, -1])   fp32
  D[h]    ~ N(0, 1)                                   fp32
  h0      zeros, or N(0, 0.1^2) per element           fp32

All draws use a CPU ``torch.Generator`` seeded explicitly, in the fixed order
x, dt, A, B, C, D, h0, then are cast (round-to-nearest-even for bf16). The CPU tensors
returned are the exact values both sides consume.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str          # "fp32" or "bf16": dtype of x, dt, B, C
    h0: bool            # random initial state (True) or zeros (False)
    seed: int

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def describe(self) -> dict:
        return {
            "workload": self.name, "batch": self.batch, "seqlen": self.seqlen,
            "nheads": self.nheads, "headdim": self.headdim, "dstate": self.dstate,
            "ngroups": self.ngroups, "chunk": self.chunk, "dtype": self.dtype,
            "h0": "N(0,0.1^2)" if self.h0 else "zeros", "seed": self.seed,
        }


# The five Mamba-2-shaped workloads (the second one in two input dtypes), and the
# benchmark shape of the article's "Mamba-2 forward pass performance benchmarks" section.
WORKLOADS = {
    "tiny-fp32": Workload("tiny-fp32", 1, 256, 2, 16, 16, 1, 64, "fp32", False, 1000),
    "small-fp32": Workload("small-fp32", 2, 2048, 24, 64, 64, 1, 64, "fp32", True, 1001),
    "small-bf16": Workload("small-bf16", 2, 2048, 24, 64, 64, 1, 64, "bf16", True, 1001),
    "780m-bf16": Workload("780m-bf16", 4, 4096, 48, 64, 128, 1, 256, "bf16", False, 1002),
    "2.7b-bf16": Workload("2.7b-bf16", 2, 16384, 80, 64, 128, 1, 256, "bf16", False, 1003),
    "long-bf16": Workload("long-bf16", 1, 65536, 80, 64, 256, 8, 256, "bf16", True, 1004),
    # the one shape the article's benchmark section spells out (batch 4, 16K tokens, 8 heads
    # of one group, dstate 128, headdim 64, chunk 128): only 32 (batch, head) pairs
    "h8-t128-bf16": Workload("h8-t128-bf16", 4, 16384, 8, 64, 128, 1, 128, "bf16", False, 1005),
}


def torch_dtype(name: str) -> torch.dtype:
    if name == "bf16":
        return torch.bfloat16
    if name == "fp32":
        return torch.float32
    raise ValueError(f"unknown input dtype {name!r}")


def make_inputs(w: Workload, *, seed: int | None = None, zero_D: bool = False) -> dict:
    """Draw one workload's inputs on the CPU. Returns x, dt, A, B, C, D, h0 (h0 may be None)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    return draw(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                torch_dtype(w.dtype), g, random_h0=w.h0, zero_D=zero_D)


def draw(batch, seqlen, nheads, headdim, dstate, ngroups, dtype, gen, *, random_h0=False,
         zero_D=False, dt_range=(1e-3, 1e-1), A_range=(1.0, 16.0)) -> dict:
    """Draw inputs of an arbitrary shape with the distributions listed in the module doc."""
    f32 = torch.float32
    x = torch.randn((batch, seqlen, nheads, headdim), generator=gen, dtype=f32)
    lo, hi = math.log(dt_range[0]), math.log(dt_range[1])
    dt = torch.exp(torch.rand((batch, seqlen, nheads), generator=gen, dtype=f32) * (hi - lo) + lo)
    alo, ahi = math.log(A_range[0]), math.log(A_range[1])
    A = -torch.exp(torch.rand((nheads,), generator=gen, dtype=f32) * (ahi - alo) + alo)
    scale = 1.0 / math.sqrt(dstate)
    B = torch.randn((batch, seqlen, ngroups, dstate), generator=gen, dtype=f32) * scale
    C = torch.randn((batch, seqlen, ngroups, dstate), generator=gen, dtype=f32) * scale
    D = torch.randn((nheads,), generator=gen, dtype=f32)
    if zero_D:
        D = torch.zeros_like(D)
    h0 = None
    if random_h0:
        h0 = torch.randn((batch, nheads, headdim, dstate), generator=gen, dtype=f32) * 0.1
    return {
        "x": x.to(dtype), "dt": dt.to(dtype), "A": A, "B": B.to(dtype), "C": C.to(dtype),
        "D": D, "h0": h0,
    }


def draw_cotangents(batch, seqlen, nheads, headdim, dstate, gen) -> dict:
    """Seeded incoming gradients for the backward pass: dy [b, L, h, P] and dfinal
    [b, h, P, S], both fp32 N(0, 1)."""
    f32 = torch.float32
    return {"dy": torch.randn((batch, seqlen, nheads, headdim), generator=gen, dtype=f32),
            "dfinal": torch.randn((batch, nheads, headdim, dstate), generator=gen, dtype=f32)}
