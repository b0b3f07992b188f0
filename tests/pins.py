"""Pins for the oracle: checks against facts that the pages and the mathematics fix.

Each ``pin_*`` takes ``fwd`` (a callable with the signature of ``oracle.forward``) and
raises AssertionError when ``fwd`` disagrees with the fact it pins. They are run on the
real oracle in ``test_oracle_pins.py`` and on deliberately broken copies of it in
``test_oracle_mutants.py`` (each planted mistake must trip at least one pin).

Sources of truth (page "Accelerating Mamba-2 with High-Performance Forward Pass Kernels
in NVIDIA CUDA Tile"):
  - section "Mamba-2 architecture": the recurrence, the renaming a = A*dt, b = dt*B, the
    decay-free jump and the statement that without decay the model is causal linear
    attention, the log-space jump formula, the decayed chunk output with causal mask;
  - section "Kernel 2: fwd_pass_state": the final state may be fed back as the next
    call's initial state;
  - the grouping of heads onto B/C groups in the kernels: group = head // heads_per_group.
"""
from __future__ import annotations

import math

import numpy as np

from chunked_ref import chunked_forward
from metrics import max_rel_rms


def rand_problem(seed, bsz, L, H, P, S, G, *, h0=True, A_zero=False, D=True):
    """Small random problem with float32-exact values (the oracle reads float32)."""
    rng = np.random.default_rng(seed)
    f = np.float32
    x = rng.standard_normal((bsz, L, H, P)).astype(f)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1) + 1.0, (bsz, L, H))).astype(f)
    A = (np.zeros(H) if A_zero else -np.exp(rng.uniform(0.0, np.log(16.0), H))).astype(f)
    B = (rng.standard_normal((bsz, L, G, S)) / math.sqrt(S)).astype(f)
    C = (rng.standard_normal((bsz, L, G, S)) / math.sqrt(S)).astype(f)
    Dv = rng.standard_normal(H).astype(f) if D else None
    hh = (0.5 * rng.standard_normal((bsz, H, P, S))).astype(f) if h0 else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=Dv, h0=hh)


def _call(fwd, p, **kw):
    return fwd(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"], **kw)


# --- hand-derived two-token example ------------------------------------------------
def pin_hand_two_tokens(fwd):
    """Worked by hand from the recurrence; P=2, S=3 so the state's orientation shows.

    A = -ln 2; dt = (1, 2) so the decays are 1/2 and 1/4. h0 = [[1,0,0],[0,1,0]], D = 3.
      t=0: x=(1,2) B=(1,0,2) C=(1,1,0):
           state = h0/2 + 1*(x outer B) = [[1.5,0,2],[2,0.5,4]];  y = state.C + 3x = (4.5, 8.5)
      t=1: x=(-1,1) B=(0,1,1) C=(0,2,1):
           state = state/4 + 2*(x outer B) = [[0.375,-2,-1.5],[0.5,2.125,3]]
           y = state.C + 3x = (-8.5, 10.25)
    """
    x = np.array([[[[1, 2]], [[-1, 1]]]], np.float32)             # [1,2,1,2]
    dt = np.array([[[1.0], [2.0]]], np.float32)                   # [1,2,1]
    A = np.array([-math.log(2.0)], np.float32)
    B = np.array([[[[1, 0, 2]], [[0, 1, 1]]]], np.float32)        # [1,2,1,3]
    C = np.array([[[[1, 1, 0]], [[0, 2, 1]]]], np.float32)
    D = np.array([3.0], np.float32)
    h0 = np.array([[[[1, 0, 0], [0, 1, 0]]]], np.float32)         # [1,1,2,3]
    out = fwd(x, dt, A, B, C, D, h0)
    y_exp = np.array([[[[4.5, 8.5]], [[-8.5, 10.25]]]])
    f_exp = np.array([[[[0.375, -2.0, -1.5], [0.5, 2.125, 3.0]]]])
    # A is ln 2 rounded to fp32, so the decays are off by ~1e-9 relative.
    assert np.allclose(out["y"], y_exp, rtol=1e-7, atol=1e-7), out["y"]
    assert np.allclose(out["final"], f_exp, rtol=1e-7, atol=1e-7), out["final"]


# --- decay-free case is causal linear attention ---------------------------------------
def pin_linear_attention_A0(fwd):
    """A = 0: y = tril(C (dt o B)^T) X + C h0^T + D X and final = h0 + X^T diag(dt) B."""
    p = rand_problem(11, 2, 37, 4, 5, 6, 2, A_zero=True)
    out = _call(fwd, p)
    x, dt, B, C, D, h0 = (np.asarray(p[k], np.float64) for k in ("x", "dt", "B", "C", "D", "h0"))
    bsz, L, H, P = x.shape
    hpg = H // B.shape[2]
    for b in range(bsz):
        for h in range(H):
            g = h // hpg
            Kb = dt[b, :, h][:, None] * B[b, :, g, :]           # keys b_t = dt_t B_t
            Q = C[b, :, g, :]
            V = x[b, :, h, :]
            scores = np.tril(Q @ Kb.T)                          # causal, diagonal kept
            y_ref = scores @ V + Q @ h0[b, h].T + D[h] * V
            f_ref = h0[b, h] + V.T @ Kb
            assert max_rel_rms(out["y"][b, :, h, :], y_ref) < 1e-13
            assert max_rel_rms(out["final"][b, h], f_ref) < 1e-13


# --- closed forms -----------------------------------------------------------------------
def pin_zero_B(fwd):
    """B = 0: the state only decays: y_t = e^{sum_{k<=t} a_k} C_t h0^T + D x_t."""
    p = rand_problem(12, 1, 23, 3, 4, 5, 1)
    p["B"] = np.zeros_like(p["B"])
    out = _call(fwd, p)
    x, dt, A, C, D, h0 = (np.asarray(p[k], np.float64) for k in ("x", "dt", "A", "C", "D", "h0"))
    for h in range(3):
        decay = np.exp(np.cumsum(A[h] * dt[0, :, h]))
        y_ref = decay[:, None] * (C[0, :, 0, :] @ h0[0, h].T) + D[h] * x[0, :, h, :]
        assert max_rel_rms(out["y"][0, :, h, :], y_ref) < 1e-13
        assert max_rel_rms(out["final"][0, h], decay[-1] * h0[0, h]) < 1e-13


def pin_zero_dt(fwd):
    """dt = 0: no decay and no input, so y = C h0^T + D x and the state stays h0."""
    p = rand_problem(13, 1, 9, 2, 3, 4, 1)
    p["dt"] = np.zeros_like(p["dt"])
    out = _call(fwd, p)
    x, C, D, h0 = (np.asarray(p[k], np.float64) for k in ("x", "C", "D", "h0"))
    for h in range(2):
        y_ref = C[0, :, 0, :] @ h0[0, h].T + D[h] * x[0, :, h, :]
        assert max_rel_rms(out["y"][0, :, h, :], y_ref) < 1e-14
        assert np.array_equal(out["final"][0, h], h0[0, h])


def pin_geometric_series(fwd):
    """Scalar state, constant decay q = e^{A dt}, x = B = 1: h_t = q^{t+1} h0 + dt (1-q^{t+1})/(1-q)."""
    L = 50
    dtv, Av, h0v, Cv = 0.25, -0.75, 2.0, 1.5
    x = np.ones((1, L, 1, 1), np.float32)
    dt = np.full((1, L, 1), dtv, np.float32)
    A = np.array([Av], np.float32)
    B = np.ones((1, L, 1, 1), np.float32)
    C = np.full((1, L, 1, 1), Cv, np.float32)
    h0 = np.array([[[[h0v]]]], np.float32)
    out = fwd(x, dt, A, B, C, None, h0)
    q = math.exp(Av * dtv)
    t = np.arange(L) + 1.0
    h = q ** t * h0v + dtv * (1 - q ** t) / (1 - q)
    assert max_rel_rms(out["y"][0, :, 0, 0], Cv * h) < 1e-13
    assert abs(out["final"][0, 0, 0, 0] - h[-1]) < 1e-13 * abs(h[-1])


# --- agreement with the page's chunked algebra ---------------------------------------
def pin_chunked_algebra(fwd):
    """Token recurrence == chunked evaluation (jump formula + decayed output), any chunk size."""
    p = rand_problem(14, 2, 67, 4, 6, 5, 2)
    out = _call(fwd, p)
    for T in (1, 8, 16, 64):
        ref = chunked_forward(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"], T)
        assert max_rel_rms(out["y"], ref["y"]) < 1e-12, T
        assert max_rel_rms(out["final"], ref["final"]) < 1e-12, T


# --- exact invariants --------------------------------------------------------------------
def pin_split_resume(fwd):
    """Running [0, L) equals running [0, L1) and then [L1, L) from the returned final state."""
    p = rand_problem(15, 2, 40, 3, 4, 5, 1)
    full = _call(fwd, p)
    L1 = 17
    a = {k: (v[:, :L1] if k in ("x", "dt", "B", "C") else v) for k, v in p.items()}
    first = _call(fwd, a)
    b = {k: (v[:, L1:] if k in ("x", "dt", "B", "C") else v) for k, v in p.items()}
    b["h0"] = first["final"].astype(np.float32)
    # the resumed state is rounded to fp32 to re-enter the oracle, so compare closely
    second = _call(fwd, b)
    assert np.array_equal(full["y"][:, :L1], first["y"])
    assert max_rel_rms(second["y"], full["y"][:, L1:]) < 1e-6
    assert max_rel_rms(second["final"], full["final"]) < 1e-6


def pin_linearity(fwd):
    """y and the final state are jointly linear in (x, h0); scaling by 2 is exact in fp."""
    p = rand_problem(16, 1, 21, 2, 3, 4, 1)
    out = _call(fwd, p)
    q = dict(p)
    q["x"] = p["x"] * np.float32(2)
    q["h0"] = p["h0"] * np.float32(2)
    out2 = _call(fwd, q)
    assert np.array_equal(out2["y"], 2 * out["y"])
    assert np.array_equal(out2["final"], 2 * out["final"])


def pin_group_broadcast(fwd):
    """ngroups = G equals ngroups = H with each head's group's B, C copied to it."""
    H, G = 6, 3
    p = rand_problem(17, 1, 19, H, 3, 4, G)
    out = _call(fwd, p)
    idx = np.arange(H) // (H // G)
    q = dict(p)
    q["B"] = p["B"][:, :, idx, :]
    q["C"] = p["C"][:, :, idx, :]
    out2 = _call(fwd, q)
    assert np.array_equal(out["y"], out2["y"])
    assert np.array_equal(out["final"], out2["final"])


def pin_head_permutation(fwd):
    """With one group, permuting heads (and their A, D, dt, x, h0) permutes the outputs."""
    p = rand_problem(18, 2, 13, 5, 3, 4, 1)
    out = _call(fwd, p)
    perm = np.array([3, 0, 4, 1, 2])
    q = dict(p)
    q["x"] = p["x"][:, :, perm]
    q["dt"] = p["dt"][:, :, perm]
    q["A"] = p["A"][perm]
    q["D"] = p["D"][perm]
    q["h0"] = p["h0"][:, perm]
    out2 = _call(fwd, q)
    assert np.array_equal(out2["y"], out["y"][:, :, perm])
    assert np.array_equal(out2["final"], out["final"][:, perm])


def pin_emitted_states(fwd):
    """The state emitted at token k*T is the final state of the run on tokens [0, k*T)."""
    p = rand_problem(19, 1, 48, 2, 3, 4, 1)
    T = 16
    out = _call(fwd, p, emit_every=T)
    assert np.array_equal(out["states"][:, :, 0], p["h0"].astype(np.float64))
    for k in range(1, 3):
        pre = {kk: (v[:, :k * T] if kk in ("x", "dt", "B", "C") else v) for kk, v in p.items()}
        assert np.array_equal(out["states"][:, :, k], _call(fwd, pre)["final"])


ALL_PINS = [
    pin_hand_two_tokens,
    pin_linear_attention_A0,
    pin_zero_B,
    pin_zero_dt,
    pin_geometric_series,
    pin_chunked_algebra,
    pin_split_resume,
    pin_linearity,
    pin_group_broadcast,
    pin_head_permutation,
    pin_emitted_states,
]
