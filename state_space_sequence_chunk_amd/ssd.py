"""Python binding of the C ABI in include/ssd.h (argument marshalling only).

Every function here forwards device pointers of torch tensors and the current HIP
stream to the shared library built from ``csrc/``; all computation happens in the HIP
kernels. When the library is missing or cannot be loaded, calls raise -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libssd_mi355x.so")

SSD_F32, SSD_BF16 = 0, 1
STATUS = {0: "SSD_OK", 1: "SSD_ERR_NULL", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_DTYPE",
          4: "SSD_ERR_UNSUPPORTED", 5: "SSD_ERR_WORKSPACE", 6: "SSD_ERR_ALIGN", 7: "SSD_ERR_HIP",
          8: "SSD_ERR_TOO_LARGE"}
# Bytes of the scratch array behind ssd_forward_noalloc (SSD_NOALLOC_SCRATCH_BYTES in ssd.h).
NOALLOC_SCRATCH_BYTES = 256 << 20

# Entry points declared in include/ssd.h.
EXPORTS = ("ssd_status_string", "ssd_validate_shape", "ssd_forward_workspace_bytes",
           "ssd_state_pass_workspace_bytes", "ssd_chunk_cumsum", "ssd_state_pass",
           "ssd_state_scan", "ssd_chunk_out", "ssd_forward", "ssd_decode_step", "ssd_backward_workspace_bytes",
           "ssd_backward", "ssd_state_pass_segmented_workspace_bytes", "ssd_state_pass_segmented",
           "ssd_chunk_out_segmented", "ssd_segment_plan", "ssd_forward_noalloc",
           "ssd_chunk_out_plan")
# HBM stream probes declared in include/ssd_probe.h (measurement only).
PROBE_EXPORTS = ("ssd_probe_read", "ssd_probe_write", "ssd_probe_copy", "ssd_probe_mix")


class SSDError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS.get(code, code)} ({msg})")
        self.code = code


class ssd_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("in_dtype", ctypes.c_int32),
                ("states_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_lib = None


def load_library():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"HIP library not built: {LIB_PATH} is missing. Build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` or "
            "`python state_space_sequence_chunk_amd/build.py`.")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    sp = ctypes.POINTER(ssd_shape)
    lib.ssd_status_string.argtypes = [i32]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_validate_shape.argtypes = [sp]
    lib.ssd_forward_workspace_bytes.argtypes = [sp, ctypes.POINTER(sz)]
    lib.ssd_state_pass_workspace_bytes.argtypes = [sp, ctypes.POINTER(sz)]
    lib.ssd_chunk_cumsum.argtypes = [sp, vp, vp, vp, vp, vp]
    lib.ssd_state_pass.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssd_state_scan.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_chunk_out.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_forward.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssd_forward_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_decode_step.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_backward_workspace_bytes.argtypes = [sp, ctypes.POINTER(sz)]
    lib.ssd_backward.argtypes = [sp] + [vp] * 17 + [sz, vp]
    lib.ssd_state_pass_segmented_workspace_bytes.argtypes = [sp, ctypes.POINTER(sz)]
    lib.ssd_state_pass_segmented.argtypes = [sp] + [vp] * 9 + [sz, vp]
    lib.ssd_chunk_out_segmented.argtypes = [sp] + [vp] * 9 + [sz, vp]
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.ssd_segment_plan.argtypes = [sp, i32p, i32p, i32p]
    lib.ssd_chunk_out_plan.argtypes = [sp, i32p, i32p, ctypes.POINTER(ctypes.c_double)]
    lib.ssd_probe_read.argtypes = [vp, sz, vp, i32, i32, vp]
    lib.ssd_probe_write.argtypes = [vp, sz, i32, i32, vp]
    lib.ssd_probe_copy.argtypes = [vp, vp, sz, i32, i32, vp]
    lib.ssd_probe_mix.argtypes = [vp, sz, vp, sz, i32, i32, vp]
    for name in EXPORTS[1:] + PROBE_EXPORTS:
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def _check(code: int, where: str):
    if code != 0:
        msg = load_library().ssd_status_string(code).decode()
        raise SSDError(code, where, msg)


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return SSD_BF16
    if dt == torch.float32:
        return SSD_F32
    raise ValueError(f"unsupported dtype {dt}")


def _code(dt):
    return dt if isinstance(dt, int) else dtype_code(dt)


def make_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, in_dtype,
               states_dtype=None, out_dtype=None) -> ssd_shape:
    """Shape struct; states default to the input dtype, y to fp32."""
    ind = _code(in_dtype)
    std = ind if states_dtype is None else _code(states_dtype)
    outd = SSD_F32 if out_dtype is None else _code(out_dtype)
    return ssd_shape(int(batch), int(seqlen), int(nheads), int(headdim), int(dstate),
                     int(ngroups), int(chunk), ind, std, outd, 0)


def shape_of(x: torch.Tensor, B: torch.Tensor, chunk: int, states_dtype=None,
             out_dtype=None) -> ssd_shape:
    """Shape struct from x [b, L, h, P] and B [b, L, g, S]."""
    b, L, H, P = x.shape
    G, S = B.shape[2], B.shape[3]
    return make_shape(b, L, H, P, S, G, chunk, x.dtype, states_dtype, out_dtype)


def _p(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the SSD library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def validate_shape(shape: ssd_shape) -> int:
    return int(load_library().ssd_validate_shape(ctypes.byref(shape)))


def forward_workspace_bytes(shape: ssd_shape) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().ssd_forward_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)),
           "ssd_forward_workspace_bytes")
    return int(n.value)


def state_pass_workspace_bytes(shape: ssd_shape) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().ssd_state_pass_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)),
           "ssd_state_pass_workspace_bytes")
    return int(n.value)


def ssd_chunk_cumsum(shape, dt, A, G, dt_t=None, stream=None):
    _check(load_library().ssd_chunk_cumsum(ctypes.byref(shape), _p(dt), _p(A), _p(G), _p(dt_t),
                                           _stream(stream)), "ssd_chunk_cumsum")


def ssd_state_pass(shape, x, A, B, G, dt_t, h0, states, final_state, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().ssd_state_pass(ctypes.byref(shape), _p(x), _p(A), _p(B), _p(G), _p(dt_t),
                                         _p(h0), _p(states), _p(final_state), _p(workspace),
                                         nbytes, _stream(stream)), "ssd_state_pass")


def ssd_state_scan(shape, x, A, B, dt_t, h0, states, final_state, stream=None):
    _check(load_library().ssd_state_scan(ctypes.byref(shape), _p(x), _p(A), _p(B), _p(dt_t),
                                         _p(h0), _p(states), _p(final_state), _stream(stream)),
           "ssd_state_scan")


def ssd_chunk_out(shape, x, B, C, G, dt_t, states, D, y, stream=None):
    _check(load_library().ssd_chunk_out(ctypes.byref(shape), _p(x), _p(B), _p(C), _p(G),
                                        _p(dt_t), _p(states), _p(D), _p(y), _stream(stream)),
           "ssd_chunk_out")


def state_pass_segmented_workspace_bytes(shape: ssd_shape) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().ssd_state_pass_segmented_workspace_bytes(ctypes.byref(shape),
                                                                   ctypes.byref(n)),
           "ssd_state_pass_segmented_workspace_bytes")
    return int(n.value)


def segment_plan(shape: ssd_shape):
    """(heads per workgroup, chunks per segment, segments) of the segmented state pass;
    raises SSDError (SSD_ERR_UNSUPPORTED) for shapes without a plan."""
    h, k, n = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load_library().ssd_segment_plan(ctypes.byref(shape), ctypes.byref(h),
                                           ctypes.byref(k), ctypes.byref(n)),
           "ssd_segment_plan")
    return int(h.value), int(k.value), int(n.value)


def chunk_out_plan(shape: ssd_shape):
    """(heads per workgroup, interaction tiles shared, executed matrix-core flops per launch)
    of the output kernel ssd_forward launches for the shape."""
    h, sh, fl = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_double(0.0)
    _check(load_library().ssd_chunk_out_plan(ctypes.byref(shape), ctypes.byref(h),
                                             ctypes.byref(sh), ctypes.byref(fl)),
           "ssd_chunk_out_plan")
    return int(h.value), bool(sh.value), float(fl.value)


def ssd_state_pass_segmented(shape, x, A, B, G, dt_t, h0, seg_relative_states, final_state,
                             workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().ssd_state_pass_segmented(
        ctypes.byref(shape), _p(x), _p(A), _p(B), _p(G), _p(dt_t), _p(h0),
        _p(seg_relative_states), _p(final_state), _p(workspace), nbytes, _stream(stream)),
        "ssd_state_pass_segmented")


def ssd_chunk_out_segmented(shape, x, B, C, G, dt_t, D, seg_relative_states, y, workspace,
                            stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().ssd_chunk_out_segmented(
        ctypes.byref(shape), _p(x), _p(B), _p(C), _p(G), _p(dt_t), _p(D),
        _p(seg_relative_states), _p(y), _p(workspace), nbytes, _stream(stream)),
        "ssd_chunk_out_segmented")


def ssd_forward(shape, x, dt, A, B, C, D, h0, y, final_state, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().ssd_forward(ctypes.byref(shape), _p(x), _p(dt), _p(A), _p(B), _p(C),
                                      _p(D), _p(h0), _p(y), _p(final_state), _p(workspace),
                                      nbytes, _stream(stream)), "ssd_forward")


def ssd_forward_noalloc(shape, x, dt, A, B, C, D, h0, y, final_state, stream=None):
    """ssd_forward without a workspace: the library's own per-device scratch array holds
    the intermediates (no allocation; calls that overlap on one GPU race)."""
    _check(load_library().ssd_forward_noalloc(ctypes.byref(shape), _p(x), _p(dt), _p(A), _p(B),
                                              _p(C), _p(D), _p(h0), _p(y), _p(final_state),
                                              _stream(stream)), "ssd_forward_noalloc")


def ssd_decode_step(shape, x, dt, A, B, C, D, state, y, stream=None):
    _check(load_library().ssd_decode_step(ctypes.byref(shape), _p(x), _p(dt), _p(A), _p(B),
                                          _p(C), _p(D), _p(state), _p(y), _stream(stream)),
           "ssd_decode_step")


def probe_read(src, sink, *, mode=0, workgroups=0, stream=None):
    """Stream `src` (a contiguous device tensor) through a read-only kernel."""
    _check(load_library().ssd_probe_read(_p(src), src.numel() * src.element_size(), _p(sink),
                                         mode, workgroups, _stream(stream)), "ssd_probe_read")


def probe_write(dst, *, mode=0, workgroups=0, stream=None):
    _check(load_library().ssd_probe_write(_p(dst), dst.numel() * dst.element_size(), mode,
                                          workgroups, _stream(stream)), "ssd_probe_write")


def probe_copy(src, dst, *, mode=0, workgroups=0, stream=None):
    if src.numel() * src.element_size() != dst.numel() * dst.element_size():
        raise ValueError("probe_copy: src and dst sizes differ")
    _check(load_library().ssd_probe_copy(_p(src), _p(dst), src.numel() * src.element_size(),
                                         mode, workgroups, _stream(stream)), "ssd_probe_copy")


def probe_mix(src, read_bytes, dst, write_bytes, *, mode=0, workgroups=0, stream=None):
    """Read read_bytes of src and write write_bytes of dst in one pass (see ssd_probe.h)."""
    if read_bytes > src.numel() * src.element_size() or write_bytes > dst.numel() * dst.element_size():
        raise ValueError("probe_mix: sizes exceed the buffers")
    _check(load_library().ssd_probe_mix(_p(src), read_bytes, _p(dst), write_bytes, mode,
                                        workgroups, _stream(stream)), "ssd_probe_mix")


def decode_step(x, dt, A, B, C, D, state, *, stream=None):
    """One token for every (batch, head): x [b, h, P], dt [b, h], B/C [b, g, S]; `state`
    (fp32 [b, h, P, S], e.g. ssd_forward's final state) is updated in place. Returns y
    (fp32 [b, h, P])."""
    b, H, P = x.shape
    sh = make_shape(b, 1, H, P, B.shape[2], B.shape[1], 1, x.dtype, torch.float32)
    y = torch.empty((b, H, P), dtype=torch.float32, device=x.device)
    ssd_decode_step(sh, x, dt, A, B, C, D, state, y, stream)
    return y


def backward_workspace_bytes(shape: ssd_shape) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().ssd_backward_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)),
           "ssd_backward_workspace_bytes")
    return int(n.value)


def ssd_backward(shape, x, dt, A, B, C, D, h0, dy, dfinal, dx, ddt, dA, dB, dC, dD, dh0,
                 workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().ssd_backward(ctypes.byref(shape), _p(x), _p(dt), _p(A), _p(B), _p(C),
                                       _p(D), _p(h0), _p(dy), _p(dfinal), _p(dx), _p(ddt),
                                       _p(dA), _p(dB), _p(dC), _p(dD), _p(dh0), _p(workspace),
                                       nbytes, _stream(stream)), "ssd_backward")


def backward(x, dt, A, B, C, D, h0, dy, dfinal=None, *, chunk, stream=None):
    """Gradients of sum(dy * y) + sum(dfinal * final) (fp32 tensors, input layouts):
    returns dict dx, ddt, dA, dB, dC, dD, dh0."""
    sh = shape_of(x, B, chunk)
    b, L, H, P = x.shape
    S = B.shape[3]
    f32 = dict(dtype=torch.float32, device=x.device)
    out = {"dx": torch.empty(x.shape, **f32), "ddt": torch.empty(dt.shape, **f32),
           "dA": torch.empty(A.shape, **f32), "dB": torch.empty(B.shape, **f32),
           "dC": torch.empty(C.shape, **f32), "dD": torch.empty((H,), **f32),
           "dh0": torch.empty((b, H, P, S), **f32)}
    ws = torch.empty(backward_workspace_bytes(sh), dtype=torch.uint8, device=x.device)
    ssd_backward(sh, x, dt, A, B, C, D, h0, dy, dfinal, out["dx"], out["ddt"], out["dA"],
                 out["dB"], out["dC"], out["dD"], out["dh0"], ws, stream)
    return out


class Forward:
    """Holds the output and workspace buffers of one problem size and runs ssd_forward.

    torch supplies the device memory; the call itself is one C-ABI invocation.
    """

    def __init__(self, x, B, chunk, states_dtype=None, device=None, out_dtype=None):
        self.shape = shape_of(x, B, chunk, states_dtype, out_dtype)
        dev = device or x.device
        b, L, H, P = x.shape
        S = B.shape[3]
        ydt = torch.bfloat16 if self.shape.out_dtype == SSD_BF16 else torch.float32
        self.y = torch.empty((b, L, H, P), dtype=ydt, device=dev)
        self.final = torch.empty((b, H, P, S), dtype=torch.float32, device=dev)
        self.workspace = torch.empty(forward_workspace_bytes(self.shape), dtype=torch.uint8,
                                     device=dev)

    def __call__(self, x, dt, A, B, C, D=None, h0=None, stream=None):
        ssd_forward(self.shape, x, dt, A, B, C, D, h0, self.y, self.final, self.workspace,
                    stream)
        return self.y, self.final


class ForwardGraph:
    """ssd_forward on fixed input buffers, recorded once in a HIP graph (through
    torch.cuda.CUDAGraph) and replayed: a replay is one graph launch instead of one launch
    per kernel, which is most of the time of a small problem. Every replay reads the input
    tensors given here (update them in place between replays) and writes the same y and
    final tensors. The forward pass records no memset and allocates nothing, so the graph
    holds only its kernels."""

    def __init__(self, x, dt, A, B, C, D=None, h0=None, *, chunk, states_dtype=None,
                 out_dtype=None):
        self.fwd = Forward(x, B, chunk, states_dtype, out_dtype=out_dtype)
        self.args = (x, dt, A, B, C, D, h0)
        # one call outside the capture (kernel attributes are set on first use)
        self.fwd(*self.args)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.fwd(*self.args, stream=torch.cuda.current_stream())

    @property
    def y(self):
        return self.fwd.y

    @property
    def final(self):
        return self.fwd.final

    def replay(self):
        self.graph.replay()
        return self.fwd.y, self.fwd.final


def forward(x, dt, A, B, C, D=None, h0=None, *, chunk, states_dtype=None, out_dtype=None,
            stream=None):
    """One-shot forward pass; returns (y [b, L, h, P] in out_dtype (fp32 by default),
    final state fp32 [b, h, P, S])."""
    f = Forward(x, B, chunk, states_dtype, out_dtype=out_dtype)
    return f(x, dt, A, B, C, D, h0, stream)
