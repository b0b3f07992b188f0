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


def _blocks(H: int, G: int, heads: int):
    """Head ranges [h0, h1) of at most ``heads`` heads that keep whole B/C groups (with
    one group, any range does)."""
    hpg = H // G
    if G > 1:
        heads = max(hpg, heads // hpg * hpg)
    return [(h0, min(H, h0 + heads)) for h0 in range(0, H, heads)]


def full_errors(y, fin, cpu: dict, *, D="given", heads: int = 16):
    """Every element of y [b, L, h, P] and of the final state [b, h, P, S] (GPU tensors)
    against the fp64 oracle, which runs on blocks of heads so that host memory stays
    bounded. Returns max|got - ref| / rms(ref) of y and of the final state, and the
    rms-relative error of y, each over the whole tensor."""
    H = cpu["A"].shape[0]
    G = cpu["B"].shape[2]
    hpg = H // G
    Dv = cpu["D"] if D == "given" else D
    acc = {"y_max": 0.0, "y_ref2": 0.0, "y_err2": 0.0, "y_n": 0,
           "f_max": 0.0, "f_ref2": 0.0, "f_n": 0}
    for h0, h1 in _blocks(H, G, heads):
        g0, g1 = h0 // hpg, (h1 - 1) // hpg + 1
        ref = oracle.forward(cpu["x"][:, :, h0:h1], cpu["dt"][:, :, h0:h1], cpu["A"][h0:h1],
                             cpu["B"][:, :, g0:g1], cpu["C"][:, :, g0:g1],
                             None if Dv is None else Dv[h0:h1],
                             None if cpu["h0"] is None else cpu["h0"][:, h0:h1])
        gy = np64(y[:, :, h0:h1])
        e = gy - ref["y"]
        acc["y_max"] = max(acc["y_max"], float(np.max(np.abs(e))))
        acc["y_ref2"] += float(np.sum(ref["y"] * ref["y"]))
        acc["y_err2"] += float(np.sum(e * e))
        acc["y_n"] += e.size
        if not np.isfinite(gy).all():
            acc["y_max"] = float("inf")
        del gy, e
        gf = np64(fin[:, h0:h1])
        ef = gf - ref["final"]
        acc["f_max"] = max(acc["f_max"], float(np.max(np.abs(ef))))
        acc["f_ref2"] += float(np.sum(ref["final"] * ref["final"]))
        acc["f_n"] += ef.size
        del ref, gf, ef
    y_rms = (acc["y_ref2"] / acc["y_n"]) ** 0.5
    f_rms = (acc["f_ref2"] / acc["f_n"]) ** 0.5
    return {"y": acc["y_max"] / y_rms,
            "y_rms_rel": (acc["y_err2"] / acc["y_n"]) ** 0.5 / y_rms,
            "final": acc["f_max"] / f_rms if f_rms > 0 else (0.0 if acc["f_max"] == 0 else
                                                             float("inf"))}


def bf16_state_bound(cpu: dict, s_ref, chunk: int, K=None):
    """Elementwise bound for bf16 chunk-initial states against the oracle's s_ref
    [b, H, nC, P, S]. One rounding to nearest even moves a value v by at most half an ulp,
    which is at most 2^-8 |v| (v just above a power of two); so 2^-8 |s_ref|, plus 1e-3
    rms(s_ref) for the fp32 arithmetic before it. With a segment plan of K chunks per
    segment, a chunk past the first segment is completed as bf16(L_c + f S_in) from the
    bf16 relative state L_c = S_c - f S_in and the bf16 entering state S_in (f its exact
    decay to the chunk): the two earlier roundings add at most 2^-8 (|L_c| + f |S_in|)
    <= 2^-8 (|S_c| + 2 f |S_in|)."""
    r = float(np.sqrt(np.mean(s_ref * s_ref)))
    bound = 2.0 ** -8 * np.abs(s_ref) + 1e-3 * r
    if K:
        A = cpu["A"].double().numpy()
        dtv = cpu["dt"].double().numpy()  # [b, L, H]
        for c in range(K, s_ref.shape[2]):
            c0 = (c // K) * K
            f = np.exp(A[None, :] * dtv[:, c0 * chunk:c * chunk, :].sum(axis=1))  # [b, H]
            fs = np.abs(f[:, :, None, None] * s_ref[:, :, c0])
            bound[:, :, c] += 2.0 ** -8 * (np.abs(s_ref[:, :, c]) + 2.0 * fs)
    return bound
