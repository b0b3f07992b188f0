"""Parity of the HIP path (through the C ABI) with the fp64 oracle on the GPU."""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_common import (SSM_MAX_TOL_FP32, SSM_RMS_TOL, TOL, bf16_state_bound, dev, gpu_forward,
                        make, needs_gpu, np64, oracle_forward, reduced)
from metrics import max_rel_rms, rms_rel
from state_space_sequence_chunk_amd import inputs as gen
from state_space_sequence_chunk_amd import ssd

pytestmark = [pytest.mark.gpu, needs_gpu]

W = gen.WORKLOADS

# Sizes whose whole output the oracle computes in seconds: the two small workloads at
# full size, the three large ones on one batch row and 4 chunks (same heads per group,
# P, S, chunk and dtype). They span several 16-row tiles, chunks and groups.
SMALL = {
    "tiny-fp32": W["tiny-fp32"],
    "small-fp32": W["small-fp32"],
    "small-bf16": W["small-bf16"],
    "780m-bf16": reduced(W["780m-bf16"], batch=1, seqlen=1024),
    "2.7b-bf16": reduced(W["2.7b-bf16"], batch=1, seqlen=1024, nheads=40),
    "long-bf16": reduced(W["long-bf16"], batch=1, seqlen=1024, nheads=40),
}


def _print(msg):
    print(msg, flush=True)


# --- stage 1 --------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(SMALL))
def test_cumsum_stage(name):
    w = SMALL[name]
    cpu, d = make(w)
    sh = ssd.shape_of(d["x"], d["B"], w.chunk)
    b, L, H = d["dt"].shape
    G = torch.empty((b, H, L), dtype=torch.float32, device="cuda")
    dt_t = torch.empty_like(G)
    ssd.ssd_chunk_cumsum(sh, d["dt"], d["A"], G, dt_t)
    torch.cuda.synchronize()
    ref = oracle.chunk_cumsum_log2(cpu["dt"], cpu["A"], w.chunk)
    err = np.abs(np64(G) - ref) / (1.0 + np.abs(ref))
    _print(f"{name}: max |dG|/(1+|G|) = {err.max():.2e}")
    assert err.max() < 1e-5
    # dt in the head-major layout, widened exactly
    assert torch.equal(dt_t.cpu(), cpu["dt"].float().permute(0, 2, 1))


# Head counts that take the kernel's other load paths: bf16 with heads not a multiple of
# 8 and fp32 with heads not a multiple of 4 (element loads), and enough chunks with many
# heads that a block holds the maximum 56 heads and the last block only 16.
@pytest.mark.parametrize("dtype,batch,seqlen,nheads,chunk", [
    ("bf16", 2, 256, 12, 64), ("fp32", 1, 512, 6, 128), ("fp32", 2, 1024, 24, 256),
    ("bf16", 1, 16384, 72, 64)])
def test_cumsum_head_blocks(dtype, batch, seqlen, nheads, chunk):
    w = gen.Workload("cumsum-shape", batch, seqlen, nheads, 16, 16, 1, chunk, dtype, False, 77)
    cpu, d = make(w)
    sh = ssd.shape_of(d["x"], d["B"], chunk)
    G = torch.empty((batch, nheads, seqlen), dtype=torch.float32, device="cuda")
    dt_t = torch.empty_like(G)
    ssd.ssd_chunk_cumsum(sh, d["dt"], d["A"], G, dt_t)
    torch.cuda.synchronize()
    ref = oracle.chunk_cumsum_log2(cpu["dt"], cpu["A"], chunk)
    err = np.abs(np64(G) - ref) / (1.0 + np.abs(ref))
    _print(f"{dtype} b{batch} L{seqlen} H{nheads} T{chunk}: max |dG|/(1+|G|) = {err.max():.2e}")
    assert err.max() < 1e-5
    assert torch.equal(dt_t.cpu(), cpu["dt"].float().permute(0, 2, 1))


# --- stage 2 --------------------------------------------------------------------------
@pytest.mark.parametrize("states", ["same", "fp32"])
@pytest.mark.parametrize("name", list(SMALL))
def test_state_pass_stage(name, states):
    w = SMALL[name]
    cpu, d = make(w)
    st_dt = d["x"].dtype if states == "same" else torch.float32
    sh = ssd.shape_of(d["x"], d["B"], w.chunk, st_dt)
    b, L, H, P = d["x"].shape
    S = d["B"].shape[3]
    nC = L // w.chunk
    G = torch.empty((b, H, L), dtype=torch.float32, device="cuda")
    dt_t = torch.empty_like(G)
    ssd.ssd_chunk_cumsum(sh, d["dt"], d["A"], G, dt_t)
    states_t = torch.empty((b, H, nC, P, S), dtype=st_dt, device="cuda")
    fin = torch.empty((b, H, P, S), dtype=torch.float32, device="cuda")
    ws = torch.empty(ssd.state_pass_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    ssd.ssd_state_pass(sh, d["x"], d["A"], d["B"], G, dt_t, d["h0"], states_t, fin, ws)
    torch.cuda.synchronize()
    ref = oracle_forward(cpu, emit_every=w.chunk)
    e_fin = max_rel_rms(fin, ref["final"])
    _print(f"{name}/{states}: final max/rms {e_fin:.2e}")
    assert e_fin <= TOL[w.dtype]
    # chunk 0 is h0 itself (or zeros); compare the states that carry information
    s_ref = ref["states"]
    if not np.any(s_ref):
        return
    got = np64(states_t)
    if st_dt == torch.bfloat16:
        # Stored in bf16: the bound of one rounding, plus the roundings of the completion
        # of segment-relative states where the shape has a segment plan
        r = float(np.sqrt(np.mean(s_ref * s_ref)))
        try:
            K = ssd.segment_plan(sh)[1]
        except ssd.SSDError:
            K = None
        bound = bf16_state_bound(cpu, s_ref, w.chunk, K)
        excess = np.abs(got - s_ref) - bound
        _print(f"{name}/{states}: bf16 states, worst excess over the rounding bound "
               f"{excess.max() / r:.2e} rms")
        assert excess.max() <= 0.0
    else:
        e_st = max_rel_rms(got, s_ref)
        _print(f"{name}/{states}: chunk-initial states max/rms {e_st:.2e}")
        assert e_st <= TOL[w.dtype]


# --- stage 3 --------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(SMALL))
def test_chunk_out_stage(name):
    """chunk_out fed the oracle's chunk-initial states reproduces the oracle's y."""
    w = SMALL[name]
    cpu, d = make(w)
    sh = ssd.shape_of(d["x"], d["B"], w.chunk)
    b, L, H, P = d["x"].shape
    ref = oracle_forward(cpu, emit_every=w.chunk)
    states_t = torch.from_numpy(ref["states"]).to(d["x"].dtype).cuda().contiguous()
    G = torch.empty((b, H, L), dtype=torch.float32, device="cuda")
    dt_t = torch.empty_like(G)
    ssd.ssd_chunk_cumsum(sh, d["dt"], d["A"], G, dt_t)
    y = torch.empty((b, L, H, P), dtype=torch.float32, device="cuda")
    ssd.ssd_chunk_out(sh, d["x"], d["B"], d["C"], G, dt_t, states_t, d["D"], y)
    torch.cuda.synchronize()
    e = max_rel_rms(y, ref["y"])
    _print(f"{name}: y max/rms {e:.2e}")
    assert e <= TOL[w.dtype]


# --- whole forward pass ---------------------------------------------------------------
@pytest.mark.parametrize("name", list(SMALL))
def test_forward_all_elements(name):
    w = SMALL[name]
    cpu, d = make(w)
    y, fin = gpu_forward(w, d)
    ref = oracle_forward(cpu)
    ey, ef = max_rel_rms(y, ref["y"]), max_rel_rms(fin, ref["final"])
    _print(f"{name}: y max/rms {ey:.2e}  final max/rms {ef:.2e}")
    assert np.isfinite(np64(y)).all()
    assert ey <= TOL[w.dtype] and ef <= TOL[w.dtype]


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_ssm_only(name):
    """D = 0: the skip term (about 99% of y) cannot mask an error in the state path."""
    w = SMALL[name]
    cpu, d = make(w, zero_D=True)
    y, _ = gpu_forward(w, d, D=None)
    ref = oracle_forward(cpu)
    er = rms_rel(y, ref["y"])
    em = max_rel_rms(y, ref["y"])
    _print(f"{name}: SSM-only rms-rel {er:.2e} max/rms {em:.2e}")
    assert er <= SSM_RMS_TOL[w.dtype]
    if w.dtype == "fp32":
        assert em <= SSM_MAX_TOL_FP32


# --- invariants and edge cases ---------------------------------------------------------
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_chunk_size_invariance(chunk, dtype):
    w = gen.Workload("inv", 1, 512, 8, 64, 64, 2, chunk, dtype, True, 2024)
    cpu, d = make(w)
    y, fin = gpu_forward(w, d)
    ref = oracle_forward(cpu)
    ey, ef = max_rel_rms(y, ref["y"]), max_rel_rms(fin, ref["final"])
    _print(f"chunk {chunk} {dtype}: y {ey:.2e} final {ef:.2e}")
    assert ey <= TOL[dtype] and ef <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_split_resume(dtype):
    """Forward over [0, L) against forward over [0, L1) then [L1, L) from the returned
    final state, L1 a chunk boundary. fp32 inputs (the two-kernel state pass): bit for
    bit. bf16 inputs take the segmented state pass, whose one-pass run forms the later
    chunk states as (state from the segment's start) + (decayed state entering it) while
    the resumed run starts from the fp32 h0, so the rounding differs: both runs within the
    parity bound of the oracle and of each other."""
    w = gen.Workload("split", 2, 1024, 4, 64, 128, 1, 256, dtype, True, 7)
    cpu, d = make(w)
    y, fin = gpu_forward(w, d)
    L1 = 512
    d1 = {k: (v[:, :L1].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in d.items()}
    d2 = {k: (v[:, L1:].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in d.items()}
    y1, f1 = gpu_forward(w, d1)
    d2["h0"] = f1
    y2, f2 = gpu_forward(w, d2)
    ys = torch.cat([y1, y2], dim=1)
    if dtype == "fp32":
        assert torch.equal(ys, y)
        assert torch.equal(f2, fin)
        return
    ref = oracle_forward(cpu)
    for got in (ys, y):
        assert max_rel_rms(got, ref["y"]) <= TOL[dtype]
    for got in (f2, fin):
        assert max_rel_rms(got, ref["final"]) <= TOL[dtype]
    assert max_rel_rms(ys, y) <= TOL[dtype] and max_rel_rms(f2, fin) <= TOL[dtype]


def test_run_to_run_bitwise_deterministic():
    w = SMALL["2.7b-bf16"]
    _, d = make(w)
    y1, f1 = gpu_forward(w, d)
    y1, f1 = y1.clone(), f1.clone()
    y2, f2 = gpu_forward(w, d)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_extreme_decay_does_not_overflow(dtype):
    """A = -16 and dt = 0.1 everywhere: masked exponents reach about +590 in log2 units
    over a 256-token chunk. They must be selected away, never reach y as inf or NaN."""
    w = gen.Workload("stress", 1, 1024, 8, 64, 128, 1, 256, dtype, True, 99)
    cpu, d = make(w)
    cpu["A"] = torch.full_like(cpu["A"], -16.0)
    cpu["dt"] = torch.full_like(cpu["dt"], 0.1)
    d["A"], d["dt"] = dev(cpu["A"]), dev(cpu["dt"])
    y, fin = gpu_forward(w, d)
    assert bool(torch.isfinite(y).all()) and bool(torch.isfinite(fin).all())
    ref = oracle_forward(cpu)
    assert max_rel_rms(y, ref["y"]) <= TOL[dtype]
    assert max_rel_rms(fin, ref["final"]) <= TOL[dtype]


def test_optional_h0_and_D():
    w = SMALL["small-bf16"]
    _, d = make(w)
    z_h0 = torch.zeros_like(d["h0"])
    z_D = torch.zeros_like(d["D"])
    y_a, f_a = gpu_forward(w, d, h0=None, D=None)
    y_a, f_a = y_a.clone(), f_a.clone()
    y_b, f_b = gpu_forward(w, d, h0=z_h0, D=z_D)
    assert torch.equal(y_a, y_b) and torch.equal(f_a, f_b)


def test_groups_match_replicated_heads():
    """ngroups = 8 equals ngroups = nheads with each group's B, C copied to its heads."""
    w = gen.Workload("grp", 1, 512, 16, 64, 64, 8, 128, "bf16", True, 5)
    _, d = make(w)
    y, fin = gpu_forward(w, d)
    y, fin = y.clone(), fin.clone()
    idx = torch.arange(16, device="cuda") // 2
    d2 = dict(d)
    d2["B"] = d["B"][:, :, idx].contiguous()
    d2["C"] = d["C"][:, :, idx].contiguous()
    y2, f2 = gpu_forward(w, d2)
    assert torch.equal(y, y2) and torch.equal(fin, f2)


def test_error_status_raises():
    w = SMALL["tiny-fp32"]
    _, d = make(w)
    with pytest.raises(ssd.SSDError):
        ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=96)


# --- bf16 y (throughput option) ---------------------------------------------------------
@pytest.mark.parametrize("name", ["small-bf16", "2.7b-bf16", "long-bf16"])
def test_bf16_y_is_fp32_y_rounded(name):
    w = SMALL[name]
    cpu, d = make(w)
    y32, f32 = gpu_forward(w, d)
    y16, f16 = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=w.chunk,
                           out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert y16.dtype == torch.bfloat16
    # the same fp32 value, rounded once to nearest even; the final state is unaffected
    assert torch.equal(y16, y32.to(torch.bfloat16)) and torch.equal(f16, f32)
    ref = oracle_forward(cpu)
    e_max = max_rel_rms(np64(y16), ref["y"])
    e_rms = rms_rel(np64(y16), ref["y"])
    _print(f"{name}: bf16 y max/rms {e_max:.2e} rms-rel {e_rms:.2e} (fp32 y bound 2e-2 not claimed)")
    assert e_rms <= 5e-3

