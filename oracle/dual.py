"""Quadratic ("dual", masked-attention) form of the Mamba-2 SSD layer, float64.

TEST INFRASTRUCTURE (see the package docstring).  Unrolling the recurrence
S_t = a_t S_{t-1} + dt_t B_t x_t^T, y_t = S_t^T C_t + D x_t gives

    y_t = sum_{s <= t} L[t, s] (C_t . B_s) dt_s x_s + D x_t,
    L[t, s] = exp(sum_{r = s+1}^{t} dt_r A)   (s <= t),   0 otherwise,

i.e. causal linear attention with a per-head decay mask (the structured
state-space duality behind Mamba-2).  O(L^2) per head: tiny inputs only.
"""
from __future__ import annotations

import numpy as np


def ssd_fwd_dual(x, dt, A, B, C, D):
    x, dt, A, B, C, D = (np.asarray(a, dtype=np.float64) for a in (x, dt, A, B, C, D))
    b, L, H, P = x.shape
    G = B.shape[2]
    hpg = H // G
    y = np.empty_like(x)
    t_idx = np.arange(L)
    causal = t_idx[:, None] >= t_idx[None, :]
    for h in range(H):
        g = h // hpg
        for bb in range(b):
            lg = dt[bb, :, h] * A[h]                 # log decay per step
            cum = np.concatenate([[0.0], np.cumsum(lg)])
            # sum_{r=s+1}^{t} lg_r = cum[t+1] - cum[s+1]
            expo = cum[1:][:, None] - cum[1:][None, :]
            Lm = np.where(causal, np.exp(np.where(causal, expo, 0.0)), 0.0)
            CB = C[bb, :, g, :] @ B[bb, :, g, :].T   # [t, s]
            M = Lm * CB
            y[bb, :, h, :] = M @ (dt[bb, :, h, None] * x[bb, :, h, :]) + D[h] * x[bb, :, h, :]
    return y
