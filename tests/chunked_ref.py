"""Independent fp64 chunked evaluation of the SSD forward pass (a pin for the oracle).

This is written from the page's chunk algebra, not from the token recurrence: page
"Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA Tile",
section "Mamba-2 architecture", the log-space jump formula for the state after a chunk
and the decayed chunk-output formula with the causal mask. Per chunk, with g the
inclusive cumulative sum of a = A*dt inside the chunk (natural-log units here, no base-2
trick):

    Y       = diag(e^g) C S^T + ((C B^T) o e^{g_i - g_j} o M) diag(dt) X + D X
    S_next  = e^{g_last} S + X^T diag(dt o e^{g_last - g}) B          (S stored P x S)

M is the lower triangle including the diagonal. Masked exponents are removed by
selection before exponentiation. A partial last chunk is just a shorter chunk.
"""
from __future__ import annotations

import numpy as np


def chunked_forward(x, dt, A, B, C, D, h0, chunk):
    x = np.asarray(x, np.float64)
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    bsz, L, H, P = x.shape
    G, S = B.shape[2], B.shape[3]
    hpg = H // G
    Dv = np.zeros(H) if D is None else np.asarray(D, np.float64)
    y = np.zeros((bsz, L, H, P))
    final = np.zeros((bsz, H, P, S))
    for b in range(bsz):
        for h in range(H):
            g = h // hpg
            state = np.zeros((P, S)) if h0 is None else np.array(h0[b, h], np.float64)
            for c0 in range(0, L, chunk):
                c1 = min(L, c0 + chunk)
                n = c1 - c0
                X = x[b, c0:c1, h, :]
                Bc = B[b, c0:c1, g, :]
                Cc = C[b, c0:c1, g, :]
                dtc = dt[b, c0:c1, h]
                gcum = np.cumsum(A[h] * dtc)
                ii, jj = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
                keep = ii >= jj
                expo = np.where(keep, gcum[:, None] - gcum[None, :], 0.0)
                decay = np.where(keep, np.exp(expo), 0.0)
                W = (Cc @ Bc.T) * decay * dtc[None, :]
                Y = np.exp(gcum)[:, None] * (Cc @ state.T) + W @ X + Dv[h] * X
                y[b, c0:c1, h, :] = Y
                wlast = dtc * np.exp(gcum[-1] - gcum)
                state = np.exp(gcum[-1]) * state + (X * wlast[:, None]).T @ Bc
            final[b, h] = state
    return {"y": y, "final": final}
