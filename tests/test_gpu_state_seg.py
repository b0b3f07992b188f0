"""The segmented state pass (ssd_state_pass_segmented + ssd_chunk_out_segmented, which ssd_forward takes
for bf16 inputs with bf16 states at headdim 64, dstate 64, 128 or 256) against the fp64
oracle on the GPU.

The shapes are chosen so that the library's segment plan differs between them: 1 to 4
heads per workgroup, 2 to 11 chunks per segment, both workgroup forms, a short last segment, a partial last
chunk, a single partial chunk, groups, with and without h0. Every element of y and of the
final state is compared."""
import numpy as np
import pytest
import torch

from gpu_common import SSM_RMS_TOL, TOL, bf16_state_bound, make, needs_gpu, oracle_forward
from metrics import max_rel_rms, rms_rel
from state_space_sequence_chunk_amd import inputs as gen
from state_space_sequence_chunk_amd import ssd

pytestmark = [pytest.mark.gpu, needs_gpu]


def _w(name, batch, seqlen, nheads, ngroups, dstate, chunk, h0, seed):
    return gen.Workload(name, batch, seqlen, nheads, 64, dstate, ngroups, chunk, "bf16", h0, seed)


# (plan the library picks for the shape: heads per workgroup x chunks per segment, segments;
# dstate 64 and 128 run 4-wave workgroups two per CU, dstate 256 8-wave ones)
CASES = {
    # 1 x 2, 8 segments; the last chunk holds 160 of 256 tokens
    "ragged-1x2": _w("ragged-1x2", 1, 4000, 10, 1, 128, 256, True, 11),
    # 1 x 2, 12 segments; chunk 128, two groups, partial last chunk
    "groups-1x2": _w("groups-1x2", 2, 3000, 12, 2, 128, 128, True, 12),
    # 1 x 2, 64 segments; chunk 64
    "t64-1x2": _w("t64-1x2", 1, 8192, 8, 1, 128, 64, False, 13),
    # 1 x 5, 4 segments; dstate 64; partial last chunk
    "s64-1x5": _w("s64-1x5", 3, 5000, 36, 1, 64, 256, False, 14),
    # 2 x 4, 8 segments
    "nh2-2x4": _w("nh2-2x4", 4, 8192, 32, 1, 128, 256, False, 15),
    # 2 x 11, 3 segments, the last of 10 chunks; dstate 64, chunk 128
    "short-seg-2x11": _w("short-seg-2x11", 8, 4096, 40, 1, 64, 128, True, 16),
    # 3 x 8, 8 segments; four groups, dstate 64, chunk 64
    "nh3-3x8": _w("nh3-3x8", 4, 4096, 48, 4, 64, 64, True, 17),
    # 4 x 8, 8 segments; dstate 64, chunk 64
    "nh4-4x8": _w("nh4-4x8", 2, 4096, 128, 1, 64, 64, False, 19),
    # 2 x 4, 4 segments; four groups, chunk 128
    "groups4-2x4": _w("groups4-2x4", 16, 2048, 48, 4, 128, 128, True, 20),
    # 1 x 2, one segment of two chunks; two groups
    "one-seg": _w("one-seg", 2, 512, 8, 2, 128, 256, True, 25),
    # one partial chunk: one segment
    "one-chunk": _w("one-chunk", 1, 200, 4, 1, 128, 256, True, 18),
    # dstate 256 (the long-context layer's per-head shape), 8-wave workgroups: 2 x 3 with
    # two 128-token sub-blocks per chunk; four groups
    "s256-2x3": _w("s256-2x3", 2, 4096, 40, 4, 256, 256, True, 21),
    # dstate 256, 1 x 2, sub-blocks, partial last chunk, no h0
    "s256-ragged-1x2": _w("s256-ragged-1x2", 1, 4000, 20, 2, 256, 256, False, 22),
    # dstate 256 at chunk 128 (one step per chunk and head) and chunk 64 (4-wave form)
    "s256-t128-1x3": _w("s256-t128-1x3", 2, 2048, 20, 2, 256, 128, True, 23),
    "s256-t64-1x2": _w("s256-t64-1x2", 1, 3000, 10, 1, 256, 64, True, 24),
}


def _print(msg):
    print(msg, flush=True)


def _forward(w, d, D="given"):
    Dv = d["D"] if D == "given" else D
    y, fin = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], Dv, d["h0"], chunk=w.chunk)
    torch.cuda.synchronize()
    return y, fin


@pytest.mark.parametrize("name", list(CASES))
def test_forward_segmented_all_elements(name):
    w = CASES[name]
    cpu, d = make(w)
    _print(f"{name}: {w}")
    y, fin = _forward(w, d)
    ref = oracle_forward(cpu)
    ey, ef = max_rel_rms(y, ref["y"]), max_rel_rms(fin, ref["final"])
    _print(f"{name}: y max/rms {ey:.2e}  final max/rms {ef:.2e}")
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"]


@pytest.mark.parametrize("name", ["ragged-1x2", "short-seg-2x11", "nh3-3x8", "s256-2x3"])
def test_forward_segmented_ssm_only(name):
    """D = 0: the state path alone, where the skip term cannot hide an error."""
    w = CASES[name]
    cpu, d = make(w, zero_D=True)
    _print(f"{name}: SSM only")
    y, fin = _forward(w, d)
    ref = oracle_forward(cpu)
    e = rms_rel(y, ref["y"])
    _print(f"{name}: SSM-only y rms-rel {e:.2e}")
    assert e <= SSM_RMS_TOL["bf16"]


def test_staged_segmented_equals_forward():
    """ssd_state_pass_segmented -> ssd_chunk_out_segmented gives ssd_forward's y and final
    state bit for bit (the same kernels in the same order)."""
    w = CASES["short-seg-2x11"]
    cpu, d = make(w)
    y1, f1 = _forward(w, d)
    sh = ssd.shape_of(d["x"], d["B"], w.chunk)
    b, L, H, P = d["x"].shape
    S = d["B"].shape[3]
    nC = -(-L // w.chunk)
    f32 = dict(dtype=torch.float32, device="cuda")
    st = torch.empty((b, H, nC, P, S), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((b, H, P, S), **f32)
    y = torch.empty((b, L, H, P), **f32)
    G = torch.empty((b, H, L), **f32)
    dtt = torch.empty((b, H, L), **f32)
    ws = torch.empty(ssd.state_pass_segmented_workspace_bytes(sh), dtype=torch.uint8,
                     device="cuda")
    ssd.ssd_chunk_cumsum(sh, d["dt"], d["A"], G, dtt)
    ssd.ssd_state_pass_segmented(sh, d["x"], d["A"], d["B"], G, dtt, d["h0"], st, fin, ws)
    ssd.ssd_chunk_out_segmented(sh, d["x"], d["B"], d["C"], G, dtt, d["D"], st, y, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y1) and torch.equal(fin, f1)


@pytest.mark.parametrize("name", ["short-seg-2x11", "ragged-1x2", "groups4-2x4", "s256-2x3",
                                  "s256-t64-1x2", "one-seg"])
def test_boundary_stages_compose_to_forward(name):
    """The boundary's three stages, ssd_chunk_cumsum -> ssd_state_pass -> ssd_chunk_out,
    give ssd_forward's y and final state bit for bit: ssd_state_pass completes the
    segment-relative states to the true chunk-initial ones with the arithmetic the output
    kernel uses for the same sum, and both routes form G with the same routine. The
    states it returns are the true ones (against the oracle, within bf16 rounding)."""
    w = CASES[name]
    cpu, d = make(w)
    y1, f1 = _forward(w, d)
    sh = ssd.shape_of(d["x"], d["B"], w.chunk)
    b, L, H, P = d["x"].shape
    S = d["B"].shape[3]
    nC = -(-L // w.chunk)
    f32 = dict(dtype=torch.float32, device="cuda")
    G = torch.empty((b, H, L), **f32)
    dtt = torch.empty((b, H, L), **f32)
    st = torch.empty((b, H, nC, P, S), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((b, H, P, S), **f32)
    y = torch.empty((b, L, H, P), **f32)
    ws = torch.empty(max(1, ssd.state_pass_workspace_bytes(sh)), dtype=torch.uint8,
                     device="cuda")
    ssd.ssd_chunk_cumsum(sh, d["dt"], d["A"], G, dtt)
    ssd.ssd_state_pass(sh, d["x"], d["A"], d["B"], G, dtt, d["h0"], st, fin, ws)
    ssd.ssd_chunk_out(sh, d["x"], d["B"], d["C"], G, dtt, st, d["D"], y)
    torch.cuda.synchronize()
    same_y, same_f = bool(torch.equal(y, y1)), bool(torch.equal(fin, f1))
    _print(f"{name} (plan {ssd.segment_plan(sh)}): staged == forward: y {same_y}, final {same_f}")
    assert same_y and same_f
    # (a completed state S_c = bf16(L_c + 2^{D_c} S_in) carries the roundings of L_c and
    # S_in as well as its own)
    ref = oracle_forward(cpu, emit_every=w.chunk)["states"]
    got = st.double().cpu().numpy()
    bound = bf16_state_bound(cpu, ref, w.chunk, ssd.segment_plan(sh)[1])
    r = float(np.max(np.abs(got - ref) / bound))
    _print(f"{name}: true states, worst error / bound {r:.3f}")
    assert r <= 1.0


def _within_bf16_rounding(got, ref):
    """Every element within bf16's round-to-nearest bound (half an ulp: 2^-8 of the value)
    plus 1e-4 of the rms for the fp32 arithmetic before the rounding; returns the worst
    ratio of error to that bound."""
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4 * np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(got - ref) / bound))


def test_segmented_recorded_states_are_segment_relative():
    """ssd_state_pass_segmented's recorded states: the true chunk-initial state minus the part
    carried in from before the segment. In the first segment (which starts from h0) they
    are the true states; at the first chunk of every later segment they are zero."""
    w = CASES["ragged-1x2"]  # two chunks per segment
    cpu, d = make(w)
    sh = ssd.shape_of(d["x"], d["B"], w.chunk)
    b, L, H, P = d["x"].shape
    S = d["B"].shape[3]
    nC = -(-L // w.chunk)
    st = torch.empty((b, H, nC, P, S), dtype=torch.bfloat16, device="cuda")
    G = torch.empty((b, H, L), dtype=torch.float32, device="cuda")
    dtt = torch.empty_like(G)
    ws = torch.empty(ssd.state_pass_segmented_workspace_bytes(sh), dtype=torch.uint8,
                     device="cuda")
    ssd.ssd_chunk_cumsum(sh, d["dt"], d["A"], G, dtt)
    ssd.ssd_state_pass_segmented(sh, d["x"], d["A"], d["B"], G, dtt, d["h0"], st, None, ws)
    torch.cuda.synchronize()
    ref = oracle_forward(cpu, emit_every=w.chunk)
    true = ref["states"]  # [b, H, nC, P, S] fp64: the state entering each chunk
    got = st.double().cpu().numpy()
    # chunks 0 and 1 form segment 0 (h0 included): the true states, to bf16 rounding
    r = _within_bf16_rounding(got[:, :, :2], true[:, :, :2])
    _print(f"segment 0 states: worst error / bf16 rounding bound {r:.3f}")
    assert r <= 1.0
    # the first chunk of each later segment records the zero state
    assert np.all(got[:, :, 2::2] == 0.0)
    # the second chunk of a segment records that segment's first chunk's own increment:
    # true S_{c+1} - 2^{g_c} S_c, with g_c the chunk's total log2 decay
    A = cpu["A"].double().numpy()
    dtv = cpu["dt"].double().numpy()  # [b, L, H]
    T = w.chunk
    for c in range(2, nC - 1, 2):
        a = np.exp(A[None, :] * dtv[:, c * T:(c + 1) * T, :].sum(axis=1))  # [b, H]
        inc = true[:, :, c + 1] - a[:, :, None, None] * true[:, :, c]
        r = _within_bf16_rounding(got[:, :, c + 1], inc)
        _print(f"chunk {c + 1}: worst error / bf16 rounding bound {r:.3f}")
        assert r <= 1.0, (c, r)
