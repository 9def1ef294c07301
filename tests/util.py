"""Shared test helpers: GPU runs of libssd and oracle references on one seeded draw."""
from __future__ import annotations

import numpy as np

NAMES_IN = ["x", "dt", "A", "B", "C", "D"]
GRADS = ["dx", "ddt", "dA", "dB", "dC", "dD"]


def max_rel(got, ref) -> float:
    """max|got - ref| / max|ref| in float64 (absolute error when ref is all zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.isfinite(got).all():
        return float("inf")
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    return float(num / den) if den > 0 else float(num)


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_gpu(inp, chunk, device="cuda"):
    """Forward + backward through libssd; returns (outputs dict of numpy float64, ctx)."""
    import torch
    from state_space_model_mamba2_amd import ssd

    dev = ssd.to_device(inp, device)
    y, fs, ctx = ssd.fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], chunk)
    g = ssd.bwd(dev["dy"], ctx)
    torch.cuda.synchronize()
    out = dict(y=to_np(y), final_state=to_np(fs))
    out.update({k: to_np(v) for k, v in g.items()})
    return out, ctx


def run_oracle(inp, nthreads=0):
    from oracle import seq

    f = {k: inp.as_f64(k) for k in NAMES_IN + ["dy"]}
    y, fs = seq.ssd_fwd(*(f[k] for k in NAMES_IN), nthreads=nthreads)
    g = seq.ssd_bwd(*(f[k] for k in NAMES_IN), f["dy"], nthreads=nthreads)
    return dict(y=y, final_state=fs, **g)
