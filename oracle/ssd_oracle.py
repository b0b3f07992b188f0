"""ctypes loader for the C oracle plus the cumulative-decay definition -- TEST INFRASTRUCTURE.

See ``oracle/__init__.py`` for who may use this module. It depends only on numpy and the
C standard library; it imports nothing from the GPU package.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_SRC_GRAD = os.path.join(_HERE, "ssd_oracle_grad.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_OUT_DIR, "libssd_oracle.so")

_lib = None


def library_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain -O2, IEEE semantics, no fast-math)."""
    if not force and not _stale():
        return _LIB
    os.makedirs(_OUT_DIR, exist_ok=True)
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-std=c99", "-Wall", "-o", tmp, _SRC, _SRC_GRAD, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _stale() -> bool:
    return not os.path.exists(_LIB) or any(
        os.path.getmtime(_LIB) < os.path.getmtime(src) for src in (_SRC, _SRC_GRAD))


def _load():
    global _lib
    if _lib is None:
        if _stale():
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        f = lib.ssd_oracle_forward
        i64 = ctypes.c_int64
        vp = ctypes.c_void_p
        f.argtypes = [i64, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp,
                      ctypes.c_int]
        f.restype = ctypes.c_int
        f = lib.ssd_oracle_forward_f64
        f.argtypes = [i64] * 6 + [vp] * 9 + [ctypes.c_int]
        f.restype = ctypes.c_int
        f = lib.ssd_oracle_backward
        f.argtypes = [i64] * 6 + [vp] * 16 + [ctypes.c_int]
        f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _np32(a):
    """float32 numpy view of an array-like; torch tensors (any device) are widened first."""
    if hasattr(a, "detach"):  # a torch tensor: widen to float32 on the host
        a = a.detach().float().cpu().numpy()
    return np.asarray(a, dtype=np.float32)


def _f32(a, shape, name):
    a = np.ascontiguousarray(_np32(a))
    if tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(a.shape)}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def forward(x, dt, A, B, C, D=None, h0=None, *, ngroups=None, emit_every=None,
            nthreads=None, want_y=True):
    """Token-by-token fp64 recurrence.

    Shapes: x [b, L, h, P], dt [b, L, h], A [h], B/C [b, L, g, S], D [h] or None,
    h0 [b, h, P, S] or None. Returns a dict with ``y`` [b, L, h, P] (float64, or None
    when ``want_y`` is False), ``final`` [b, h, P, S] and, when ``emit_every`` is given,
    ``states`` [b, h, ceil(L/emit_every), P, S]: the state before token k*emit_every.
    Inputs are converted to float32 first; callers pass values that are exact in fp32.
    """
    x = _np32(x)
    if x.ndim != 4:
        raise ValueError("x must be [batch, seqlen, nheads, headdim]")
    bsz, L, H, P = x.shape
    B = _np32(B)
    if B.ndim != 4:
        raise ValueError("B must be [batch, seqlen, ngroups, dstate]")
    G, S = B.shape[2], B.shape[3]
    if ngroups is not None and ngroups != G:
        raise ValueError("ngroups disagrees with B")
    x32 = _f32(x, (bsz, L, H, P), "x")
    dt32 = _f32(dt, (bsz, L, H), "dt")
    A32 = _f32(A, (H,), "A")
    B32 = _f32(B, (bsz, L, G, S), "B")
    C32 = _f32(C, (bsz, L, G, S), "C")
    D32 = None if D is None else _f32(D, (H,), "D")
    h032 = None if h0 is None else _f32(h0, (bsz, H, P, S), "h0")
    y = np.empty((bsz, L, H, P), np.float64) if want_y else None
    final = np.empty((bsz, H, P, S), np.float64)
    states = None
    ee = 0
    if emit_every is not None:
        ee = int(emit_every)
        states = np.empty((bsz, H, -(-L // ee), P, S), np.float64)
    nt = _default_threads() if nthreads is None else int(nthreads)
    rc = _load().ssd_oracle_forward(bsz, L, H, P, S, G, _ptr(x32), _ptr(dt32), _ptr(A32),
                                    _ptr(B32), _ptr(C32), _ptr(D32), _ptr(h032), _ptr(y),
                                    _ptr(final), ee, _ptr(states), nt)
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    out = {"y": y, "final": final}
    if states is not None:
        out["states"] = states
    return out


def forward_pairs(pairs, x, dt, A, B, C, D=None, h0=None, *, nthreads=None):
    """Run the recurrence on the listed (batch, head) pairs of a full-size problem.

    The inputs are array-likes with ``__getitem__`` (numpy arrays, or anything whose
    slices convert with ``np.asarray``), in the full layouts of ``forward``. Each pair
    becomes one independent head of a small stacked problem (batch 1, one group per
    head), which is the same recurrence. Returns ``y`` [n, L, P] and ``final``
    [n, P, S] in the order of ``pairs``.
    """
    A_np = _np32(A)
    H = A_np.shape[0]
    G = B.shape[2]
    hpg = H // G
    xs, dts, As, Bs, Cs, Ds, h0s = [], [], [], [], [], [], []
    D_np = None if D is None else _np32(D)
    for (b, h) in pairs:
        g = h // hpg
        xs.append(_np32(x[b, :, h, :]))
        dts.append(_np32(dt[b, :, h]))
        As.append(A_np[h])
        Bs.append(_np32(B[b, :, g, :]))
        Cs.append(_np32(C[b, :, g, :]))
        Ds.append(0.0 if D_np is None else D_np[h])
        if h0 is not None:
            h0s.append(_np32(h0[b, h]))
    n = len(pairs)
    xx = np.stack(xs, axis=1)[None]          # [1, L, n, P]
    dd = np.stack(dts, axis=1)[None]         # [1, L, n]
    BB = np.stack(Bs, axis=1)[None]          # [1, L, n, S]
    CC = np.stack(Cs, axis=1)[None]
    hh = None if h0 is None else np.stack(h0s, axis=0)[None]  # [1, n, P, S]
    out = forward(xx, dd, np.asarray(As, np.float32), BB, CC, np.asarray(Ds, np.float32), hh,
                  nthreads=nthreads)
    y = np.ascontiguousarray(np.transpose(out["y"][0], (1, 0, 2)))  # [n, L, P]
    return {"y": y, "final": out["final"][0]}


def chunk_cumsum_log2(dt, A, chunk):
    """Per-chunk inclusive cumulative decay in base-2 log units.

    For token t in chunk c = t // chunk:  G[b, h, t] = log2(e) * sum_{k = c*chunk}^{t} A[h]*dt[b, k, h].
    The sum restarts at every chunk (it is not a global cumulative sum); a partial last
    chunk simply ends early. Returned as float64 [b, h, L] (head-major, tokens fastest).
    """
    dt = _np32(dt).astype(np.float64)
    A = _np32(A).astype(np.float64)
    bsz, L, H = dt.shape
    a = dt * A[None, None, :]
    G = np.empty((bsz, H, L), np.float64)
    log2e = 1.0 / math.log(2.0)
    for c0 in range(0, L, chunk):
        c1 = min(L, c0 + chunk)
        run = np.zeros((bsz, H), np.float64)
        for t in range(c0, c1):
            run = run + a[:, t, :]
            G[:, :, t] = run * log2e
    return G


# --- gradients (ssd_oracle_grad.c) ----------------------------------------------------
def _np64(a):
    """float64 numpy copy of an array-like; torch tensors (any device) are widened."""
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().double().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def forward64(x, dt, A, B, C, D=None, h0=None, *, nthreads=None):
    """The recurrence with float64 inputs (values used as given, no rounding to float32),
    for finite differences. Returns {"y": [b, L, h, P], "final": [b, h, P, S]}."""
    x, dt, A, B, C, D, h0 = (_np64(v) for v in (x, dt, A, B, C, D, h0))
    bsz, L, H, P = x.shape
    G, S = B.shape[2], B.shape[3]
    y = np.empty((bsz, L, H, P), np.float64)
    fin = np.empty((bsz, H, P, S), np.float64)
    rc = _load().ssd_oracle_forward_f64(bsz, L, H, P, S, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                        _ptr(C), _ptr(D), _ptr(h0), _ptr(y), _ptr(fin),
                                        nthreads or _default_threads())
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_forward_f64 failed ({rc})")
    return {"y": y, "final": fin}


def backward(x, dt, A, B, C, D, h0, dy, dfinal=None, *, nthreads=None):
    """Gradients of sum(dy * y) + sum(dfinal * final) with respect to every input, in
    float64 (reverse-mode through the token recurrence; see ssd_oracle_grad.c).
    Returns dx, ddt, dA [h], dB, dC [b, L, g, S], dD [h] and dh0 [b, h, P, S]; dA and dD
    are summed over the batch here."""
    x, dt, A, B, C, D, h0, dy, dfinal = (_np64(v) for v in (x, dt, A, B, C, D, h0, dy, dfinal))
    bsz, L, H, P = x.shape
    G, S = B.shape[2], B.shape[3]
    dx = np.empty_like(x)
    ddt = np.empty_like(dt)
    dB = np.empty_like(B)
    dC = np.empty_like(C)
    dA_bh = np.empty((bsz, H), np.float64)
    dD_bh = np.empty((bsz, H), np.float64)
    dh0 = np.empty((bsz, H, P, S), np.float64)
    rc = _load().ssd_oracle_backward(bsz, L, H, P, S, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                     _ptr(C), _ptr(D), _ptr(h0), _ptr(dy), _ptr(dfinal),
                                     _ptr(dx), _ptr(ddt), _ptr(dA_bh), _ptr(dB), _ptr(dC),
                                     _ptr(dD_bh), _ptr(dh0), nthreads or _default_threads())
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_backward failed ({rc})")
    return {"dx": dx, "ddt": ddt, "dA": dA_bh.sum(axis=0), "dB": dB, "dC": dC,
            "dD": dD_bh.sum(axis=0), "dh0": dh0}

