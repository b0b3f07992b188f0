"""Pins of the gradient oracle, as plain functions of the oracle module (so they can also
be run against planted mistakes): finite differences of the fp64 forward, closed forms
that follow from the recurrence, and the fp64 forward being the pinned forward oracle."""
import numpy as np
import torch

from state_space_sequence_chunk_amd import inputs as gen

GRAD_OF = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "h0": "dh0"}

# (batch, L, heads, headdim, dstate, groups), elements sampled per input (None: all)
FD_CASES = [
    ((2, 7, 4, 3, 5, 2), None),        # every element of every input
    ((1, 70, 2, 2, 3, 1), 25),         # across a recompute checkpoint (every 64 tokens)
    ((1, 5, 3, 2, 4, 3), None),        # one head per group
]


def problem(batch, L, H, P, S, G, seed, h0=True):
    g = torch.Generator()
    g.manual_seed(seed)
    d = gen.draw(batch, L, H, P, S, G, torch.float32, g, random_h0=h0)
    d = {k: (None if v is None else v.double().numpy()) for k, v in d.items()}
    rng = np.random.default_rng(seed)
    wy = rng.standard_normal((batch, L, H, P))
    wf = rng.standard_normal((batch, H, P, S))
    return d, wy, wf


def _loss(o, d, wy, wf):
    out = o.forward64(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], nthreads=1)
    return float(np.sum(wy * out["y"]) + np.sum(wf * out["final"]))


def pin_forward64_is_forward(o):
    g = torch.Generator()
    g.manual_seed(3)
    d = gen.draw(2, 70, 4, 8, 16, 2, torch.bfloat16, g, random_h0=True)
    ref = o.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"])
    got = o.forward64(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"])
    assert np.array_equal(got["y"], ref["y"]) and np.array_equal(got["final"], ref["final"])


def pin_finite_differences(o, shape, sample):
    batch, L, H, P, S, G = shape
    d, wy, wf = problem(batch, L, H, P, S, G, seed=11 + L)
    gr = o.backward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], wy, wf,
                    nthreads=2)
    rng = np.random.default_rng(5)
    for name, gname in GRAD_OF.items():
        base = d[name]
        idx = np.arange(base.size)
        if sample is not None and base.size > sample:
            idx = rng.choice(base.size, sample, replace=False)
        fd = np.empty(len(idx))
        for k, i in enumerate(idx):
            v = base.flat[i]
            eps = 1e-6 * max(1.0, abs(v))
            dp = {kk: (None if vv is None else vv.copy()) for kk, vv in d.items()}
            dp[name].flat[i] = v + eps
            lp = _loss(o, dp, wy, wf)
            dp[name].flat[i] = v - eps
            lm = _loss(o, dp, wy, wf)
            fd[k] = (lp - lm) / (2 * eps)
        got = gr[gname].reshape(-1)[idx]
        scale = max(float(np.sqrt(np.mean(gr[gname] ** 2))), 1e-300)
        err = float(np.max(np.abs(got - fd))) / scale
        assert err < 1e-6, f"d{name}: {err:.2e}"


def pin_closed_forms(o):
    d, wy, wf = problem(2, 9, 4, 3, 5, 2, seed=21)
    gr = o.backward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], wy, wf)
    # D enters only as D x: dD = sum over batch, tokens and P of dy * x
    assert np.allclose(gr["dD"], np.einsum("btnp,btnp->n", wy, d["x"]), rtol=1e-13, atol=0)
    # dt = 0 freezes the state at h0: y_t = h0 C_t + D x_t, final = h0
    z = dict(d)
    z["dt"] = np.zeros_like(d["dt"])
    g0 = o.backward(z["x"], z["dt"], z["A"], z["B"], z["C"], z["D"], z["h0"], wy, wf)
    hpg = 2
    C_h = np.repeat(d["C"], hpg, axis=2)  # [b, L, h, S]
    assert np.allclose(g0["dx"], d["D"][None, None, :, None] * wy, rtol=1e-13, atol=1e-15)
    assert np.allclose(g0["dh0"], np.einsum("btnp,btns->bnps", wy, C_h) + wf, rtol=1e-12,
                       atol=1e-14)
    dC_h = np.einsum("bnps,btnp->btns", d["h0"], wy)  # per head, then summed per group
    assert np.allclose(g0["dC"], dC_h.reshape(2, 9, 2, hpg, 5).sum(axis=3), rtol=1e-12,
                       atol=1e-14)
    assert np.array_equal(g0["dB"], np.zeros_like(g0["dB"]))
    # no tokens: the final state is h0, so dh0 = dfinal and nothing else moves
    e = {k: (None if v is None else (v[:, :0] if k in ("x", "dt", "B", "C") else v))
         for k, v in d.items()}
    ge = o.backward(e["x"], e["dt"], e["A"], e["B"], e["C"], e["D"], e["h0"], wy[:, :0], wf)
    assert np.array_equal(ge["dh0"], wf) and not np.any(ge["dA"]) and not np.any(ge["dD"])


def pin_single_token(o):
    # one token, worked by hand from H = e^{a} h0 + dt x B^T, y = H C + D x (a = A dt),
    # loss = dy . y + <dfinal, H>; with Lam = dy C^T + dfinal:
    #   dx = D dy + dt Lam B,  dB = dt Lam^T x,  dC = H^T dy,  dD = dy . x,
    #   dh0 = e^{a} Lam,  ddt = x . Lam B + A e^{a} <Lam, h0>,  dA = dt e^{a} <Lam, h0>
    rng = np.random.default_rng(8)
    P, S, H = 3, 4, 2
    x = rng.standard_normal((1, 1, H, P))
    dt = rng.uniform(0.01, 0.5, (1, 1, H))
    A = -rng.uniform(1.0, 8.0, H)
    B = rng.standard_normal((1, 1, 1, S))
    C = rng.standard_normal((1, 1, 1, S))
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((1, H, P, S))
    dy = rng.standard_normal((1, 1, H, P))
    dfin = rng.standard_normal((1, H, P, S))
    g = o.backward(x, dt, A, B, C, D, h0, dy, dfin)
    b, c = B[0, 0, 0], C[0, 0, 0]
    dB = np.zeros(S)
    dC = np.zeros(S)
    for h in range(H):
        xv, dyv, d = x[0, 0, h], dy[0, 0, h], dt[0, 0, h]
        e = np.exp(A[h] * d)
        Hs = e * h0[0, h] + d * np.outer(xv, b)
        lam = np.outer(dyv, c) + dfin[0, h]
        np.testing.assert_allclose(g["dx"][0, 0, h], D[h] * dyv + d * lam @ b, rtol=1e-12)
        np.testing.assert_allclose(g["dh0"][0, h], e * lam, rtol=1e-12)
        inner = np.sum(lam * h0[0, h])
        np.testing.assert_allclose(g["ddt"][0, 0, h], xv @ lam @ b + A[h] * e * inner,
                                   rtol=1e-11)
        np.testing.assert_allclose(g["dA"][h], d * e * inner, rtol=1e-11)
        np.testing.assert_allclose(g["dD"][h], dyv @ xv, rtol=1e-12)
        dB += d * lam.T @ xv
        dC += Hs.T @ dyv
    np.testing.assert_allclose(g["dB"][0, 0, 0], dB, rtol=1e-11)
    np.testing.assert_allclose(g["dC"][0, 0, 0], dC, rtol=1e-11)


def all_grad_pins():
    """(name, callable taking the oracle module) for every pin."""
    pins = [("forward64_is_forward", pin_forward64_is_forward),
            ("closed_forms", pin_closed_forms),
            ("single_token", pin_single_token)]
    for shape, sample in FD_CASES:
        pins.append((f"finite_differences{shape}",
                     lambda o, shape=shape, sample=sample: pin_finite_differences(o, shape, sample)))
    return pins
