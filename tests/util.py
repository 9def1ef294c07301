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


def run_gpu(inp, chunk, device="cuda", states=None):
    """Forward + backward through libssd; returns (outputs dict of numpy float64, ctx).
    states: optional (initial_state, dfinal_state) float32 numpy arrays; with
    them the outputs include dinitial_state."""
    import torch
    from state_space_model_mamba2_amd import ssd

    dev = ssd.to_device(inp, device)
    s0 = dfs = None
    if states is not None:
        s0, dfs = (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device) for a in states)
    y, fs, ctx = ssd.fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], chunk, initial_state=s0)
    g = ssd.bwd(dev["dy"], ctx, dfinal_state=dfs, want_dinitial_state=states is not None)
    torch.cuda.synchronize()
    out = dict(y=to_np(y), final_state=to_np(fs))
    out.update({k: to_np(v) for k, v in g.items()})
    return out, ctx


def run_oracle(inp, nthreads=0, states=None):
    """Oracle outputs; without states the dinitial_state entry is dropped."""
    from oracle import seq

    f = {k: inp.as_f64(k) for k in NAMES_IN + ["dy"]}
    s0, dfs = (None, None) if states is None else (np.asarray(a, np.float64) for a in states)
    y, fs = seq.ssd_fwd(*(f[k] for k in NAMES_IN), initial_state=s0, nthreads=nthreads)
    g = seq.ssd_bwd(*(f[k] for k in NAMES_IN), f["dy"], initial_state=s0, dfinal_state=dfs, nthreads=nthreads)
    if states is None:
        g.pop("dinitial_state")
    return dict(y=y, final_state=fs, **g)
