"""Error metrics used by the parity tests.

``max_rel_rms(got, ref)`` = max |got - ref| / rms(ref), both widened to float64: the
largest elementwise error measured in units of the reference tensor's root mean square.
"""
from __future__ import annotations

import numpy as np


def to_np64(a):
    if hasattr(a, "detach"):
        a = a.detach().float().cpu().numpy()
    return np.asarray(a, dtype=np.float64)


def rms(a) -> float:
    a = to_np64(a)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def max_rel_rms(got, ref) -> float:
    got = to_np64(got)
    ref = to_np64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    r = rms(ref)
    d = float(np.max(np.abs(got - ref)))
    if r == 0.0:
        return 0.0 if d == 0.0 else float("inf")
    return d / r


def rms_rel(got, ref) -> float:
    got = to_np64(got)
    ref = to_np64(ref)
    r = rms(ref)
    return rms(got - ref) / r if r else (0.0 if rms(got - ref) == 0 else float("inf"))
