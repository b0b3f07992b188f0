"""Shared helpers of the GPU parity tests: seeded inputs on the device, the HIP path
through the C ABI, the oracle on the same values, and the tolerances."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from state_space_sequence_chunk_amd import inputs as gen
from state_space_sequence_chunk_amd import ssd

HAVE_GPU = torch.cuda.is_available()
needs_gpu = pytest.mark.skipif(not HAVE_GPU, reason="needs an MI355X GPU")

# Parity bounds on max|got - oracle| / rms(oracle), for y and for the final state:
# 1e-5 with fp32 inputs, 2e-2 with bf16 inputs (fp32 accumulation in both).
TOL = {"fp32": 1e-5, "bf16": 2e-2}
# Extra gate on the SSM-only output (D = 0), where the skip term cannot hide errors:
# rms-relative error, and for fp32 also max/rms.
SSM_RMS_TOL = {"fp32": 1e-5, "bf16": 1e-2}
SSM_MAX_TOL_FP32 = 1e-4


def dev(t):
    return None if t is None else t.to("cuda", non_blocking=False).contiguous()


def reduced(w: gen.Workload, *, batch=None, seqlen=None, nheads=None):
    """Same per-head shapes, dtype and distributions as ``w``, on fewer tokens/heads."""
    import dataclasses
    kw = {}
    if batch is not None:
        kw["batch"] = batch
    if seqlen is not None:
        kw["seqlen"] = seqlen
    if nheads is not None:
        kw["nheads"] = nheads
    return dataclasses.replace(w, name=w.name + "-reduced", **kw)


def make(w: gen.Workload, *, zero_D=False, seed=None):
    cpu = gen.make_inputs(w, zero_D=zero_D, seed=seed)
    return cpu, {k: dev(v) for k, v in cpu.items()}


def gpu_forward(w: gen.Workload, d: dict, *, chunk=None, states_dtype=None, D="given",
                h0="given"):
    T = chunk or w.chunk
    Dv = d["D"] if D == "given" else D
    hv = d["h0"] if h0 == "given" else h0
    y, fin = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], Dv, hv, chunk=T,
                         states_dtype=states_dtype)
    torch.cuda.synchronize()
    return y, fin


def oracle_forward(cpu: dict, *, D="given", emit_every=None):
    Dv = cpu["D"] if D == "given" else D
    return oracle.forward(cpu["x"], cpu["dt"], cpu["A"], cpu["B"], cpu["C"], Dv, cpu["h0"],
                          emit_every=emit_every)


def np64(t):
    return t.detach().double().cpu().numpy()
