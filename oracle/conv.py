"""Causal depthwise conv1d of the Mamba block, float64 -- TEST INFRASTRUCTURE.

The convolution that precedes the SSD scan in a Mamba block (the "causal
conv" whose forward and backward the LightOn page "Training Mamba Models on
AMD MI250/MI250X GPUs with Custom Kernels", section "Individual Kernels",
times on MI250).  The page gives no
formula; this is the operation's definition.  Per channel c, with a width-W
filter w[c][0..W-1], a bias and an optional activation (SiLU, z * sigmoid(z)):

    z[b, t, c] = bias[c] + sum_{k=0}^{W-1} w[c][k] * x[b, t - (W-1) + k, c]
    y[b, t, c] = act(z[b, t, c])

Causal: rows before the sequence are zero, or the W-1 rows x_prev[b][0..W-2]
(times -(W-1) .. -1) when given, which is what carries a sequence cut into
pieces.  Layout token-major, x, y [b][L][C], x_prev [b][W-1][C], w [C][W].

Backward of <dy, y>, with g = dy * act'(z) (act' = 1, or for SiLU
sigmoid(z) * (1 + z * (1 - sigmoid(z)))):

    dx[b, s, c]  = sum_k w[c][k] * g[b, s + (W-1) - k, c]   (terms inside [0, L))
    dw[c][k]     = sum_{b, t} g[b, t, c] * x[b, t - (W-1) + k, c]
    dbias[c]     = sum_{b, t} g[b, t, c]
    dx_prev      = dx at the rows -(W-1) .. -1

Plain numpy over the W taps; nothing is blocked or fused.
"""
from __future__ import annotations

import numpy as np


def _sigmoid(z):
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def _padded(x, x_prev, W):
    x = np.asarray(x, dtype=np.float64)
    b, L, C = x.shape
    prev = np.zeros((b, W - 1, C)) if x_prev is None else np.asarray(x_prev, dtype=np.float64)
    return np.concatenate([prev, x], axis=1)  # row r is time r - (W-1)


def _preact(xp, w, bias, L):
    W = w.shape[1]
    z = np.zeros((xp.shape[0], L, xp.shape[2]))
    for k in range(W):
        z += w[:, k][None, None, :] * xp[:, k:k + L, :]
    if bias is not None:
        z += np.asarray(bias, dtype=np.float64)[None, None, :]
    return z


def conv1d_fwd(x, w, bias=None, x_prev=None, silu=True):
    w = np.asarray(w, dtype=np.float64)
    W = w.shape[1]
    L = np.shape(x)[1]
    z = _preact(_padded(x, x_prev, W), w, bias, L)
    return z * _sigmoid(z) if silu else z


def conv1d_bwd(x, w, dy, bias=None, x_prev=None, silu=True):
    """Gradients (dx, dw, dbias, dx_prev) of <dy, y>."""
    w = np.asarray(w, dtype=np.float64)
    W = w.shape[1]
    b, L, C = np.shape(x)
    xp = _padded(x, x_prev, W)
    z = _preact(xp, w, bias, L)
    dy = np.asarray(dy, dtype=np.float64)
    if silu:
        s = _sigmoid(z)
        g = dy * s * (1.0 + z * (1.0 - s))
    else:
        g = dy
    dxp = np.zeros_like(xp)
    dw = np.zeros((C, W))
    for k in range(W):
        dxp[:, k:k + L, :] += w[:, k][None, None, :] * g
        dw[:, k] = np.einsum("btc,btc->c", g, xp[:, k:k + L, :])
    return dict(dx=dxp[:, W - 1:], dw=dw, dbias=g.sum(axis=(0, 1)), dx_prev=dxp[:, :W - 1])
