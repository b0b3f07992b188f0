"""The C-ABI library loads, exports every declared entry point, and rejects invalid
arguments on the host before anything is enqueued (no GPU needed)."""
import ctypes
import os
import re

import pytest

from state_space_sequence_chunk_amd import ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

pytestmark = pytest.mark.skipif(not os.path.exists(ssd.LIB_PATH),
                                reason="HIP library not built (run __graft_entry__.build())")


def declared_functions(paths=(HEADER,)):
    names = set()
    for path in paths:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"\b(ssd_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_four_stages():
    names = declared_functions()
    for n in ("ssd_chunk_cumsum", "ssd_state_pass", "ssd_chunk_out", "ssd_forward"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ssd.load_library()
    names = declared_functions(HEADERS)
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    assert sorted(ssd.EXPORTS + ssd.PROBE_EXPORTS) == names
    assert sorted(ssd.EXPORTS) == declared_functions()


def test_shape_struct_matches_header():
    # seven int64 sizes, then in_dtype, states_dtype, out_dtype, reserved (int32)
    assert ctypes.sizeof(ssd.ssd_shape) == 7 * 8 + 4 * 4
    assert ssd.ssd_shape.out_dtype.offset == 7 * 8 + 2 * 4


def shape(**kw):
    base = dict(batch=2, seqlen=512, nheads=8, headdim=64, dstate=128, ngroups=2, chunk=256,
                in_dtype=ssd.SSD_BF16, states_dtype=None, out_dtype=None)
    base.update(kw)
    return ssd.make_shape(**base)


@pytest.mark.parametrize("kw,code", [
    ({}, 0),
    (dict(batch=0), 2), (dict(seqlen=-1), 2), (dict(nheads=0), 2), (dict(ngroups=3), 2),
    (dict(seqlen=0), 0), (dict(seqlen=500), 0), (dict(seqlen=1), 0),
    (dict(chunk=96, seqlen=576), 4), (dict(chunk=32, seqlen=512), 4), (dict(chunk=0), 2),
    (dict(headdim=48), 4), (dict(dstate=96), 4), (dict(dstate=512), 4),
    (dict(in_dtype=7), 3), (dict(states_dtype=5), 3),
    (dict(headdim=16, dstate=16, chunk=64, in_dtype=ssd.SSD_F32), 0),
    (dict(out_dtype=ssd.SSD_BF16), 0), (dict(out_dtype=7), 3),
    (dict(out_dtype=ssd.SSD_BF16, states_dtype=ssd.SSD_F32), 4),
    (dict(out_dtype=ssd.SSD_BF16, in_dtype=ssd.SSD_F32, states_dtype=ssd.SSD_F32), 4),
])
def test_validate_shape(kw, code):
    assert ssd.validate_shape(shape(**kw)) == code


def test_workspace_sizes():
    s = shape(states_dtype=ssd.SSD_BF16)
    nchunks = 512 // 256
    elems = 2 * 8 * nchunks * 64 * 128
    dec = 2 * 8 * 512 * 4
    # bf16 inputs and states: the state pass is segmented; its workspace (and that of the
    # segmented pair) holds the segment buffers: at least one segment's end state (fp32) and
    # entering state (bf16) per (batch, head); the forward's adds G, dt_t and the states
    seg = ssd.state_pass_segmented_workspace_bytes(s)
    assert seg >= 2 * 8 * 64 * 128 * (4 + 2)
    assert ssd.state_pass_workspace_bytes(s) == seg
    assert ssd.forward_workspace_bytes(s) == 2 * dec + seg + elems * 2
    # fp32 states: no segment plan, the two-kernel pass's increments
    s32 = shape(states_dtype=ssd.SSD_F32)
    assert ssd.state_pass_workspace_bytes(s32) == elems * 4
    assert ssd.forward_workspace_bytes(s32) == 2 * dec + elems * 4 + elems * 4
    with pytest.raises(ssd.SSDError):
        ssd.forward_workspace_bytes(shape(ngroups=3))
    for kw in (dict(states_dtype=ssd.SSD_F32), dict(in_dtype=ssd.SSD_F32, states_dtype=ssd.SSD_F32),
               dict(headdim=128)):
        with pytest.raises(ssd.SSDError) as e:
            ssd.state_pass_segmented_workspace_bytes(shape(**kw))
        assert e.value.code == 4, kw
    # dstate 256 (128-token sub-blocks inside the kernel) has a plan at every chunk length
    for t in (64, 128, 256):
        assert ssd.state_pass_segmented_workspace_bytes(shape(dstate=256, chunk=t)) > 0
    assert ssd.state_pass_segmented_workspace_bytes(shape(seqlen=0)) == 0


def test_segment_plan_query():
    # the 2.7B layer: 2 heads per workgroup, 11 chunks per segment, 6 segments (480
    # 4-wave workgroups, two per CU)
    s = ssd.make_shape(2, 16384, 80, 64, 128, 1, 256, ssd.SSD_BF16)
    assert ssd.segment_plan(s) == (2, 11, 6)
    # the long layer at dstate 256: 2 heads x 43 chunks, 6 segments (240 workgroups)
    assert ssd.segment_plan(ssd.make_shape(1, 65536, 80, 64, 256, 8, 256, ssd.SSD_BF16)) == (2, 43, 6)
    # the 780M layer: 2 heads x 4 chunks (4 segments, 384 workgroups); the 8-head benchmark
    # shape with 128-token chunks and the small layer take one head per workgroup (no
    # shared B rows): 8 chunks, 16 segments and 4 chunks, 8 segments
    assert ssd.segment_plan(ssd.make_shape(4, 4096, 48, 64, 128, 1, 256, ssd.SSD_BF16)) == (2, 4, 4)
    assert ssd.segment_plan(ssd.make_shape(4, 16384, 8, 64, 128, 1, 128, ssd.SSD_BF16)) == (1, 8, 16)
    assert ssd.segment_plan(ssd.make_shape(2, 2048, 24, 64, 64, 1, 64, ssd.SSD_BF16)) == (1, 4, 8)
    lib = ssd.load_library()
    assert lib.ssd_segment_plan(ctypes.byref(s), None, None, None) == 0
    for kw in (dict(states_dtype=ssd.SSD_F32), dict(headdim=128), dict(seqlen=0)):
        with pytest.raises(ssd.SSDError) as e:
            ssd.segment_plan(shape(**kw))
        assert e.value.code == 4, kw
    assert lib.ssd_segment_plan(ctypes.byref(shape(ngroups=3)), None, None, None) == 2


def test_segmented_entry_points_reject_before_launch():
    lib = ssd.load_library()
    s = shape()
    f = _v(FAKE)
    need = ssd.state_pass_segmented_workspace_bytes(s)
    # x A B G dt_t h0 seg_relative_states final
    args = [f, f, f, f, f, None, f, None]
    for i in (0, 1, 2, 3, 4, 6):  # required pointers
        bad = list(args)
        bad[i] = None
        assert lib.ssd_state_pass_segmented(ctypes.byref(s), *bad, f, need, None) == 1, i
    assert lib.ssd_state_pass_segmented(ctypes.byref(s), *args, f, need - 1, None) == 5
    assert lib.ssd_state_pass_segmented(ctypes.byref(s), *args, None, need, None) == 5
    bad = list(args)
    bad[6] = _v(FAKE + 4)
    assert lib.ssd_state_pass_segmented(ctypes.byref(s), *bad, f, need, None) == 6
    s32 = shape(states_dtype=ssd.SSD_F32)
    assert lib.ssd_state_pass_segmented(ctypes.byref(s32), *args, f, need, None) == 4
    assert lib.ssd_state_pass_segmented(ctypes.byref(shape(ngroups=3)), *args, f, need, None) == 2
    # x B C G dt_t D seg_relative_states y
    oargs = [f, f, f, f, f, None, f, f]
    for i in (0, 1, 2, 3, 4, 6, 7):
        bad = list(oargs)
        bad[i] = None
        assert lib.ssd_chunk_out_segmented(ctypes.byref(s), *bad, f, need, None) == 1, i
    assert lib.ssd_chunk_out_segmented(ctypes.byref(s), *oargs, f, need - 1, None) == 5
    assert lib.ssd_chunk_out_segmented(ctypes.byref(s), *oargs, None, need, None) == 5
    assert lib.ssd_chunk_out_segmented(ctypes.byref(s32), *oargs, f, need, None) == 4
    bad = list(oargs)
    bad[3] = _v(FAKE + 4)
    assert lib.ssd_chunk_out_segmented(ctypes.byref(s), *bad, f, need, None) == 6
    # the empty sequence: the final state only (none wanted here), no launch
    e = shape(seqlen=0)
    assert lib.ssd_state_pass_segmented(ctypes.byref(e), None, f, *[None] * 6, None, 0,
                                        None) == 0
    assert lib.ssd_chunk_out_segmented(ctypes.byref(e), *[None] * 8, None, 0, None) == 0


def _round256(n):
    return (n + 255) // 256 * 256


def test_workspace_sizes_ragged_and_empty():
    # 300 tokens in chunks of 256: two chunks, the second holding 44 real tokens
    s = shape(seqlen=300, states_dtype=ssd.SSD_F32)
    elems = 2 * 8 * 2 * 64 * 128
    assert ssd.state_pass_workspace_bytes(s) == elems * 4
    dec = _round256(2 * 8 * 300 * 4)
    assert ssd.forward_workspace_bytes(s) == 2 * dec + elems * 4 + elems * 4
    e = shape(seqlen=0)
    assert ssd.state_pass_workspace_bytes(e) == 0 and ssd.forward_workspace_bytes(e) == 0


def test_empty_sequence_host_paths():
    # nothing to compute and no final state wanted: success with no launch and NULL tensors
    lib = ssd.load_library()
    e = shape(seqlen=0)
    f = _v(FAKE)
    assert lib.ssd_chunk_cumsum(ctypes.byref(e), None, f, None, None, None) == 0
    assert lib.ssd_chunk_out(ctypes.byref(e), *[None] * 8, None) == 0
    assert lib.ssd_forward(ctypes.byref(e), None, None, f, None, None, None, None, None, None,
                           None, 0, None) == 0
    assert lib.ssd_state_pass(ctypes.byref(e), None, f, None, None, None, None, None, None,
                              None, 0, None) == 0
    # A is still required
    assert lib.ssd_forward(ctypes.byref(e), *[None] * 10, 0, None) == 1


def test_null_shape_and_null_out_pointer():
    lib = ssd.load_library()
    assert lib.ssd_validate_shape(None) == 1
    assert lib.ssd_forward_workspace_bytes(ctypes.byref(shape()), None) == 1


FAKE = 1 << 20  # an aligned, never-dereferenced address: validation fails before any launch


def _v(addr):
    return ctypes.c_void_p(addr)


def test_forward_rejects_before_launch():
    lib = ssd.load_library()
    s = shape()
    need = ssd.forward_workspace_bytes(s)
    args = [_v(FAKE)] * 9  # x dt A B C D h0 y final
    # missing x
    assert lib.ssd_forward(ctypes.byref(s), None, *args[1:], _v(FAKE), need, None) == 1
    # misaligned y
    bad = list(args)
    bad[7] = _v(FAKE + 4)
    assert lib.ssd_forward(ctypes.byref(s), *bad, _v(FAKE), need, None) == 6
    # workspace too small / missing
    assert lib.ssd_forward(ctypes.byref(s), *args, _v(FAKE), need - 1, None) == 5
    assert lib.ssd_forward(ctypes.byref(s), *args, None, need, None) == 5
    # invalid shape wins over everything else
    s2 = shape(ngroups=3)
    assert lib.ssd_forward(ctypes.byref(s2), *args, _v(FAKE), need, None) == 2


def test_stage_entry_points_reject_before_launch():
    lib = ssd.load_library()
    s = shape()
    f = _v(FAKE)
    assert lib.ssd_chunk_cumsum(ctypes.byref(s), None, f, f, f, None) == 1
    assert lib.ssd_chunk_cumsum(ctypes.byref(s), f, f, _v(FAKE + 8), f, None) == 6
    need = ssd.state_pass_workspace_bytes(s)
    assert lib.ssd_state_pass(ctypes.byref(s), f, f, f, f, f, None, None, None, f, need, None) == 1
    assert lib.ssd_state_pass(ctypes.byref(s), f, None, f, f, f, None, f, None, f, need, None) == 1
    assert lib.ssd_state_pass(ctypes.byref(s), f, f, f, f, f, None, f, None, f, need - 16, None) == 5
    assert lib.ssd_chunk_out(ctypes.byref(s), f, f, f, f, f, None, None, f, None) == 1
    assert lib.ssd_chunk_out(ctypes.byref(s), f, f, f, f, f, f, _v(FAKE + 2), f, None) == 6


def test_state_scan_rejects_before_launch():
    lib = ssd.load_library()
    f = _v(FAKE)
    # x A B dt_t h0 states final
    args = [f, f, f, f, None, f, None]
    s = shape()
    for i in (0, 1, 2, 3, 5):  # required pointers
        bad = list(args)
        bad[i] = None
        assert lib.ssd_state_scan(ctypes.byref(s), *bad, None) == 1, i
    bad = list(args)
    bad[5] = _v(FAKE + 4)  # misaligned states
    assert lib.ssd_state_scan(ctypes.byref(s), *bad, None) == 6
    # shapes outside the kernel's plans: fp32 inputs, a partial last chunk, headdim 32,
    # dstate 32, the empty sequence
    for kw in (dict(in_dtype=ssd.SSD_F32, states_dtype=ssd.SSD_F32), dict(seqlen=500),
               dict(headdim=32), dict(dstate=32), dict(seqlen=0)):
        assert lib.ssd_state_scan(ctypes.byref(shape(**kw)), *args, None) == 4, kw
    assert lib.ssd_state_scan(ctypes.byref(shape(ngroups=3)), *args, None) == 2
    assert lib.ssd_state_scan(None, *args, None) == 1


def test_decode_step_rejects_before_launch():
    lib = ssd.load_library()
    f = _v(FAKE)
    args = [f] * 8  # x dt A B C D state y
    ok = shape(seqlen=1)
    # a valid call would launch: only the rejecting cases are called here
    assert lib.ssd_decode_step(ctypes.byref(shape()), *args, None) == 2  # seqlen != 1
    assert lib.ssd_decode_step(ctypes.byref(shape(seqlen=1, ngroups=3)), *args, None) == 2
    assert lib.ssd_decode_step(ctypes.byref(shape(seqlen=1, in_dtype=9)), *args, None) == 3
    assert lib.ssd_decode_step(ctypes.byref(shape(seqlen=1, headdim=48)), *args, None) == 4
    assert lib.ssd_decode_step(ctypes.byref(shape(seqlen=1, dstate=512)), *args, None) == 4
    bad = list(args)
    bad[6] = None  # state
    assert lib.ssd_decode_step(ctypes.byref(ok), *bad, None) == 1
    bad = list(args)
    bad[5] = None  # D is optional: still fails later on the misaligned y only
    bad[7] = _v(FAKE + 4)
    assert lib.ssd_decode_step(ctypes.byref(ok), *bad, None) == 6
    assert lib.ssd_decode_step(None, *args, None) == 1
    # chunk and states_dtype are not used by the decode step
    assert lib.ssd_decode_step(ctypes.byref(shape(seqlen=1, chunk=7, states_dtype=5)),
                               *[None] * 8, None) == 1


def test_status_strings():
    lib = ssd.load_library()
    for code in range(8):
        assert lib.ssd_status_string(code)
    assert lib.ssd_status_string(99) == b"unknown status"


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(ssd, "_lib", None)
    monkeypatch.setattr(ssd, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not built"):
        ssd.load_library()


def test_backward_workspace_sizes():
    # G, dt_t, chunk-initial states, gradients at the chunk ends, final state, three
    # per-token scalars, two per-(batch, head) partials, per-head dB, dC (shared groups),
    # and the per-chunk anchors of the log-decay suffix sums
    # bf16 inputs, P = 64, S = 128: the matrix-core kernels run at 128-token chunks (3 here)
    s = shape(seqlen=300)
    dec = _round256(2 * 8 * 300 * 4)
    fin = 2 * 8 * 64 * 128 * 4
    part = _round256(2 * 300 * 8 * 128 * 4)
    st = 2 * 8 * 3 * 64 * 128 * 4
    anc = _round256(st // 256)  # per-chunk anchors of the log-decay suffix sums
    want = 2 * dec + 2 * st + fin + 3 * dec + 2 * 256 + 2 * part + anc
    assert ssd.backward_workspace_bytes(s) == want
    # one head per group: the per-head partials are the outputs themselves
    s1 = shape(seqlen=300, ngroups=8)
    assert ssd.backward_workspace_bytes(s1) == want - 2 * part
    # fp32 inputs take the token walks at the caller's chunk (2 chunks of 256); the
    # backward pass ignores states_dtype and out_dtype
    st2 = 2 * 8 * 2 * 64 * 128 * 4
    want2 = 2 * dec + 2 * st2 + fin + 3 * dec + 2 * 256 + 2 * part + _round256(st2 // 256)
    for sd in (ssd.SSD_F32, ssd.SSD_BF16):
        assert ssd.backward_workspace_bytes(shape(seqlen=300, in_dtype=ssd.SSD_F32,
                                                  states_dtype=sd)) == want2
    assert ssd.backward_workspace_bytes(shape(seqlen=300, out_dtype=ssd.SSD_BF16)) == want
    assert ssd.backward_workspace_bytes(shape(seqlen=0)) == 0


def test_backward_rejects_before_launch():
    lib = ssd.load_library()
    s = shape()
    f = _v(FAKE)
    need = ssd.backward_workspace_bytes(s)
    # x dt A B C D h0 dy dfinal dx ddt dA dB dC dD dh0
    args = [f] * 16
    for i in (0, 1, 2, 3, 4, 7, 9, 10, 11, 12, 13):  # required pointers
        bad = list(args)
        bad[i] = None
        assert lib.ssd_backward(ctypes.byref(s), *bad, f, need, None) == 1, i
    bad = list(args)
    bad[10] = _v(FAKE + 4)  # misaligned ddt
    assert lib.ssd_backward(ctypes.byref(s), *bad, f, need, None) == 6
    assert lib.ssd_backward(ctypes.byref(s), *args, f, need - 1, None) == 5
    assert lib.ssd_backward(ctypes.byref(s), *args, None, need, None) == 5
    assert lib.ssd_backward(ctypes.byref(shape(ngroups=3)), *args, f, need, None) == 2
    assert lib.ssd_backward(ctypes.byref(shape(dstate=96)), *args, f, need, None) == 4
    assert lib.ssd_backward(None, *args, f, need, None) == 1
    n = ctypes.c_size_t(0)
    assert lib.ssd_backward_workspace_bytes(ctypes.byref(s), None) == 1
    assert lib.ssd_backward_workspace_bytes(ctypes.byref(shape(in_dtype=9)), ctypes.byref(n)) == 3


def test_backward_workspace_without_partials():
    # 2 x 16384 tokens, 80 heads in one group, bf16: the matrix-core kernels run at
    # 128-token chunks with all 80 heads of the group in one workgroup and write dB, dC
    # directly, so no per-head partials are reserved
    s = shape(batch=2, seqlen=16384, nheads=80, ngroups=1, chunk=256)
    dec = _round256(2 * 80 * 16384 * 4)
    st = 2 * 80 * 128 * 64 * 128 * 4
    fin = 2 * 80 * 64 * 128 * 4
    bh = _round256(2 * 80 * 4)
    anc = _round256(st // 256)
    assert ssd.backward_workspace_bytes(s) == 2 * dec + 2 * st + fin + 3 * dec + 2 * bh + anc


def test_backward_chunk_stays_within_size_limits():
    # dstate 256 has a matrix-core plan at 64-token chunks, but at 262144 tokens and 32
    # heads its fp32 chunk states would pass 2e9 elements; the backward then takes the fp32
    # token walks at the caller's 256-token chunks (a quarter of the states)
    L = 262144
    s = shape(batch=1, seqlen=L, nheads=32, ngroups=1, headdim=64, dstate=256, chunk=256)
    dec = _round256(32 * L * 4)
    st = 32 * (L // 256) * 64 * 256 * 4
    fin = 32 * 64 * 256 * 4
    bh = _round256(32 * 4)
    part = L * 32 * 256 * 4  # per-head dB, dC partials of the walks
    anc = _round256(st // 256)
    assert ssd.backward_workspace_bytes(s) == (2 * dec + 2 * st + fin + 3 * dec + 2 * bh +
                                               2 * part + anc)
    # 16 heads stay within the limit at 64-token chunks: the matrix-core plan applies, with
    # four times the chunk states
    s16 = shape(batch=1, seqlen=L, nheads=16, ngroups=1, headdim=64, dstate=256, chunk=256)
    assert ssd.backward_workspace_bytes(s16) > 2 * 16 * (L // 64) * 64 * 256 * 4


# --- HBM stream probes (include/ssd_probe.h): host-side validation only ---------------------
@pytest.mark.parametrize("call,code", [
    (lambda L: L.ssd_probe_read(None, 1024, 4096, 0, 0, None), 1),
    (lambda L: L.ssd_probe_read(4096, 0, 8192, 0, 0, None), 2),
    (lambda L: L.ssd_probe_read(4096, 1000, 8192, 0, 0, None), 2),
    (lambda L: L.ssd_probe_read(4100, 1024, 8192, 0, 0, None), 6),
    (lambda L: L.ssd_probe_read(4096, 1024, 8192, 2, 0, None), 4),
    (lambda L: L.ssd_probe_write(None, 1024, 0, 0, None), 1),
    (lambda L: L.ssd_probe_write(4096, 1024, 0, -1, None), 2),
    (lambda L: L.ssd_probe_copy(4096, 8200, 1024, 0, 0, None), 6),
    (lambda L: L.ssd_probe_copy(4096, 8192, 1024, 5, 0, None), 4),
    (lambda L: L.ssd_probe_mix(None, 1024, 8192, 1024, 0, 0, None), 1),
    (lambda L: L.ssd_probe_mix(4096, 1024, None, 16, 0, 0, None), 1),
    (lambda L: L.ssd_probe_mix(4096, 0, 8192, 0, 0, 0, None), 2),
    (lambda L: L.ssd_probe_mix(4096, 1000, 8192, 1024, 0, 0, None), 2),
    (lambda L: L.ssd_probe_mix(4104, 1024, 8192, 1024, 0, 0, None), 6),
    (lambda L: L.ssd_probe_mix(4096, 1024, 8192, 2048, 3, 0, None), 4),
])
def test_probe_argument_checks(call, code):
    assert call(ssd.load_library()) == code


# --- ssd_forward_noalloc: the size check happens on the host, before any HIP call ---------
def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define SSD_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == ssd.NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_too_large_on_host():
    lib = ssd.load_library()
    big = shape(batch=1, seqlen=65536, nheads=80, headdim=64, dstate=256, ngroups=8, chunk=256)
    assert ssd.forward_workspace_bytes(big) > ssd.NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(4096)
    rc = lib.ssd_forward_noalloc(ctypes.byref(big), p, p, p, p, p, p, p, p, p, None)
    assert rc == 8
    assert b"scratch" in lib.ssd_status_string(8)
    # the bench shape fits
    bench = shape(batch=2, seqlen=16384, nheads=80, headdim=64, dstate=128, ngroups=1, chunk=256)
    assert ssd.forward_workspace_bytes(bench) <= ssd.NOALLOC_SCRATCH_BYTES


def test_chunk_out_plan_counts_the_executed_products():
    # the 2.7B layer: 40 heads per workgroup (256 workgroups of 8 waves fill the 256 CUs
    # once), interaction tiles shared. Per workgroup: 136 lower-triangular 16x16 tiles of
    # C B^T at K = 128 (4 products of K = 32); per head: C_i . S_c for 16 row tiles x 4
    # p-tiles x 4 K-steps, and W x for the row tiles' column-tile pairs (72) x 4 p-tiles.
    # Every product is 2 x 16 x 16 x 32 flops.
    s = ssd.make_shape(2, 16384, 80, 64, 128, 1, 256, ssd.SSD_BF16)
    nh, shared, flops = ssd.chunk_out_plan(s)
    assert (nh, shared) == (40, True)
    pairs = sum(it // 2 + 1 for it in range(16))
    assert pairs == 72
    per_wg = 136 * 4 + 40 * (16 * 4 * 4 + 72 * 4)
    assert flops == per_wg * 256 * 2 * 16 * 16 * 32
    # fp32 states with bf16 inputs: the carried-state product runs on a high/low split
    s32 = ssd.make_shape(2, 16384, 80, 64, 128, 1, 256, ssd.SSD_BF16, states_dtype=ssd.SSD_F32)
    nh32, sh32, f32 = ssd.chunk_out_plan(s32)
    tiles = 136 * 4 * (1 if sh32 else nh32)
    assert f32 == (tiles + nh32 * (16 * 4 * 4 * 2 + 72 * 4)) * (2 * 16384 * 80 // (256 * nh32)) * 16384
    with pytest.raises(ssd.SSDError) as e:
        ssd.chunk_out_plan(shape(seqlen=0))
    assert e.value.code == 4
