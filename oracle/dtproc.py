"""Step-size preprocessing of the Mamba-2 SSD layer, float64 -- TEST INFRASTRUCTURE.

The layer's step is dt = softplus(dt_raw + dt_bias) with one bias per head,
softplus(z) = log(1 + e^z) (the Mamba-2 block's parameterisation that the
workloads of the Zyphra/AMD post's "Mamba-2" section are drawn from).  Its
backward is the chain rule through that map:

    d dt / d dt_raw = sigmoid(dt_raw + dt_bias),
    ddt_raw[b, t, h] = ddt[b, t, h] * sigmoid(dt_raw[b, t, h] + dt_bias[h]),
    ddt_bias[h]      = sum over b, t of ddt_raw[b, t, h].

Both are written out from that definition; the scan itself is the
sequential oracle (seq.py) applied to the resulting dt.
"""
from __future__ import annotations

import numpy as np


def softplus(z):
    z = np.asarray(z, dtype=np.float64)
    # log(1 + e^z) = max(z, 0) + log1p(e^{-|z|}), exact in either tail
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def step(dt_raw, dt_bias):
    """dt = softplus(dt_raw + dt_bias); dt_raw [b, L, H], dt_bias [H] (None: zero)."""
    z = np.asarray(dt_raw, dtype=np.float64)
    if dt_bias is not None:
        z = z + np.asarray(dt_bias, dtype=np.float64)[None, None, :]
    return softplus(z)


def step_grads(ddt, dt_raw, dt_bias):
    """(ddt_raw, ddt_bias) from the gradient ddt of the post-softplus step."""
    z = np.asarray(dt_raw, dtype=np.float64)
    if dt_bias is not None:
        z = z + np.asarray(dt_bias, dtype=np.float64)[None, None, :]
    ddt_raw = np.asarray(ddt, dtype=np.float64) * sigmoid(z)
    return ddt_raw, ddt_raw.sum(axis=(0, 1))
