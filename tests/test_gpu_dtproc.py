"""libssd with the fused step preprocessing dt = softplus(dt_raw + dt_bias).

The library takes the raw step and the per-head bias, applies the softplus
in the chunk cumsum and chains its gradient in the dl assembly; the oracle is
the plain definition (oracle/dtproc.py) around the sequential recurrence.
ddt is then the gradient w.r.t. dt_raw and ddt_bias the bias gradient.
Tolerance as elsewhere (1e-4 fp32, 2e-2 bf16 and FP8, max|gpu - ref| / max|ref|).
"""
import numpy as np
import pytest

from state_space_model_mamba2_amd import inputs
from tests.util import NAMES_IN, max_rel, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# fp8: against the oracle on the E4M3 values themselves (the kernels widen them exactly)
TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 2e-2}


def run_gpu_softplus(inp, chunk, states=None):
    from state_space_model_mamba2_amd import ssd

    dev = ssd.to_device(inp, "cuda")
    s0 = dfs = None
    if states is not None:
        s0, dfs = (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda() for a in states)
    y, fs, ctx = ssd.fwd(dev["x"], dev["dt_raw"], dev["A"], dev["B"], dev["C"], dev["D"], chunk,
                         initial_state=s0, dt_softplus=True, dt_bias=dev["dt_bias"])
    g = ssd.bwd(dev["dy"], ctx, dfinal_state=dfs, want_dinitial_state=states is not None)
    torch.cuda.synchronize()
    out = dict(y=to_np(y), final_state=to_np(fs))
    out.update({k: to_np(v) for k, v in g.items()})
    return out


def run_oracle_softplus(inp, states=None, batch=None, heads=None):
    """Oracle outputs on batch rows `batch` and heads `heads` (slices; all by default)."""
    from oracle import dtproc, seq

    bs = batch or slice(None)
    hs = heads or slice(None)
    H, G = inp.shape.nheads, inp.shape.ngroups
    hg = np.arange(H)[hs]
    groups = sorted(set((hg // (H // G)).tolist()))
    assert heads is None or len(groups) == 1 or len(hg) == H
    gs = slice(groups[0], groups[-1] + 1)
    f = {k: inp.as_f64(k) for k in NAMES_IN + ["dy", "dt_raw", "dt_bias"]}
    x, dy = f["x"][bs][:, :, hs], f["dy"][bs][:, :, hs]
    raw, bias = f["dt_raw"][bs][:, :, hs], f["dt_bias"][hs]
    B, C = f["B"][bs][:, :, gs], f["C"][bs][:, :, gs]
    A, D = f["A"][hs], f["D"][hs]
    s0 = dfs = None
    if states is not None:
        s0, dfs = (np.asarray(a, np.float64)[bs][:, hs] for a in states)
    dt = dtproc.step(raw, bias)
    y, fs = seq.ssd_fwd(x, dt, A, B, C, D, initial_state=s0)
    g = seq.ssd_bwd(x, dt, A, B, C, D, dy, initial_state=s0, dfinal_state=dfs)
    g["ddt"], g["ddt_bias"] = dtproc.step_grads(g["ddt"], raw, bias)
    if states is None:
        g.pop("dinitial_state")
    return dict(y=y, final_state=fs, **g)


CASES = [
    ("tiny_fp32", dict()),
    ("tiny_fp32", dict(batch=2, seqlen=64 * 3 + 5, nheads=4, ngroups=2)),
    ("mamba2_370m", dict(batch=2, seqlen=512, nheads=4, chunk=64, dtype="f32")),
    ("mamba2_370m", dict(batch=2, seqlen=1024, nheads=4)),
    ("mamba2_370m", dict(batch=2, seqlen=900, nheads=4)),
    ("zamba2_7b", dict(batch=1, seqlen=640, nheads=8, ngroups=2, chunk=128)),
    ("long_context", dict(seqlen=2048, nheads=16, ngroups=2)),
    # E4M3 x, B, C with the fused step, both passes (a ragged tail and two groups)
    ("mamba2_370m", dict(batch=2, seqlen=900, nheads=4, dtype="fp8")),
    ("zamba2_7b", dict(batch=1, seqlen=640, nheads=8, ngroups=2, chunk=128, dtype="fp8")),
]


def _id(case):
    s = inputs.workload(case[0], **case[1])
    return f"{s.dtype}-Q{s.chunk}-P{s.headdim}-N{s.dstate}-G{s.ngroups}-L{s.seqlen}"


@pytest.mark.parametrize("with_states", [False, True])
@pytest.mark.parametrize("case", CASES, ids=_id)
def test_softplus_parity(case, with_states):
    shape = inputs.workload(case[0], **case[1])
    print(f"[softplus] {shape} states={with_states}", flush=True)
    inp = inputs.generate(shape, seed=11)
    st = inputs.generate_states(shape, seed=11) if with_states else None
    got = run_gpu_softplus(inp, shape.chunk, st)
    ref = run_oracle_softplus(inp, st)
    assert set(got) == set(ref)
    errs = {k: max_rel(got[k], ref[k]) for k in ref}
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[shape.dtype]}
    assert not bad, f"{shape}: over tolerance: {bad}"


def test_softplus_full_size_sampled():
    """The 2.7B workload with the fused step: batch row 0 with every head, and
    all batch rows of two heads for the per-head sums (dA, dD, ddt_bias)."""
    shape = inputs.workload("mamba2_2p7b")
    print(f"[softplus full] {shape}", flush=True)
    inp = inputs.generate(shape, seed=12)
    got = run_gpu_softplus(inp, shape.chunk)
    ref = run_oracle_softplus(inp, batch=slice(0, 1))
    keys = ("y", "final_state", "dx", "ddt", "dB", "dC")
    errs = {k: max_rel(got[k][:1], ref[k]) for k in keys}
    ref2 = run_oracle_softplus(inp, heads=slice(0, 2))
    for k in ("dA", "dD", "ddt_bias"):
        errs[k] = max_rel(got[k][:2], ref2[k])
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
    assert not bad, bad
