"""FP8 (OCP E4M3) x, B, C in the forward and backward passes, on the GPU.

Parity: the library's forward and backward on E4M3 inputs against the float64
oracle on exactly those E4M3 values (the kernels widen the codes exactly, so
this measures the kernels' own arithmetic: bf16 products with fp32
accumulation, C.B^T on the FP8 matrix cores, dy and every gradient in bf16),
tolerance 2e-2 as in bf16 mode.  The end-to-end cost of storing x, B, C in
FP8 instead of bf16 is measured against the oracle on the bf16 values of the
same draws and printed; it is bounded by the CPU study in
tests/test_fp8_accuracy.py.
"""
import numpy as np
import pytest

from state_space_model_mamba2_amd import inputs
from tests.util import max_rel, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2


def run_fwd_gpu(inp, chunk, states=None):
    from state_space_model_mamba2_amd import ssd

    dev = ssd.to_device(inp, "cuda")
    s0 = torch.from_numpy(states[0]).cuda() if states is not None else None
    y, fs, _ = ssd.fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], chunk, initial_state=s0)
    torch.cuda.synchronize()
    return to_np(y), to_np(fs)


def oracle_fwd(inp, states=None, batch=slice(None)):
    from oracle import seq

    f = {k: inp.as_f64(k)[batch] if k not in ("A", "D") else inp.as_f64(k) for k in ("x", "dt", "A", "B", "C", "D")}
    s0 = None if states is None else states[0][batch].astype(np.float64)
    return seq.ssd_fwd(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], initial_state=s0)


CASES = [
    ("mamba2_370m", dict(batch=2, seqlen=1024, nheads=4)),
    ("mamba2_370m", dict(batch=2, seqlen=700, nheads=4, ngroups=2, chunk=128)),
    ("zamba2_7b", dict(batch=1, seqlen=768, nheads=8, ngroups=2)),
    ("tiny_fp32", dict(batch=2, seqlen=300, nheads=4, chunk=128)),
]


@pytest.mark.parametrize("with_states", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1].get('seqlen')}-Q{c[1].get('chunk', 256)}")
def test_fp8_forward_parity(case, with_states):
    shape = inputs.workload(case[0], **case[1]).replace(dtype="fp8")
    print(f"[fp8] {shape} states={with_states}", flush=True)
    inp = inputs.generate(shape, seed=30)
    st = inputs.generate_states(shape, seed=30) if with_states else None
    y, fs = run_fwd_gpu(inp, shape.chunk, st)
    ry, rfs = oracle_fwd(inp, st)
    e = dict(y=max_rel(y, ry), final_state=max_rel(fs, rfs))
    ref16 = inputs.generate(shape.replace(dtype="bf16"), seed=30)
    by, bfs = oracle_fwd(ref16, st)
    e16 = dict(y=max_rel(y, by), final_state=max_rel(fs, bfs))
    print(f"  vs oracle on the E4M3 values: {e}; vs oracle on the bf16 values: {e16}", flush=True)
    assert all(v <= TOL for v in e.values()), e


def test_fp8_full_size_sampled():
    shape = inputs.workload("mamba2_2p7b").replace(dtype="fp8")
    print(f"[fp8 full] {shape}", flush=True)
    inp = inputs.generate(shape, seed=31)
    y, fs = run_fwd_gpu(inp, shape.chunk)
    ry, rfs = oracle_fwd(inp, batch=slice(0, 1))
    e = dict(y=max_rel(y[:1], ry), final_state=max_rel(fs[:1], rfs))
    print(f"  {e}", flush=True)
    assert all(v <= TOL for v in e.values()), e


def run_fwd_bwd_gpu(inp, chunk, states=None):
    from state_space_model_mamba2_amd import ssd

    dev = ssd.to_device(inp, "cuda")
    s0, dfs = ((torch.from_numpy(a).cuda() for a in states) if states is not None else (None, None))
    y, fs, ctx = ssd.fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], chunk, initial_state=s0)
    g = ssd.bwd(dev["dy"], ctx, dfinal_state=dfs, want_dinitial_state=states is not None)
    torch.cuda.synchronize()
    out = dict(y=to_np(y), final_state=to_np(fs))
    out.update({k: to_np(v) for k, v in g.items()})
    return out


def oracle_fwd_bwd(inp, states=None):
    from tests.util import run_oracle

    return run_oracle(inp, states=states)


@pytest.mark.parametrize("with_states", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1].get('seqlen')}-Q{c[1].get('chunk', 256)}")
def test_fp8_backward_parity(case, with_states):
    shape = inputs.workload(case[0], **case[1]).replace(dtype="fp8")
    print(f"[fp8 bwd] {shape} states={with_states}", flush=True)
    inp = inputs.generate(shape, seed=33)
    st = inputs.generate_states(shape, seed=33) if with_states else None
    got = run_fwd_bwd_gpu(inp, shape.chunk, st)
    ref = oracle_fwd_bwd(inp, st)
    e = {k: max_rel(got[k], ref[k]) for k in ref}
    ref16 = oracle_fwd_bwd(inputs.generate(shape.replace(dtype="bf16"), seed=33), st)
    e16 = {k: max_rel(got[k], ref16[k]) for k in ref16}
    print("  vs oracle on the E4M3 values: " + " ".join(f"{k}={v:.1e}" for k, v in e.items()), flush=True)
    print("  vs oracle on the bf16 values: " + " ".join(f"{k}={v:.1e}" for k, v in e16.items()), flush=True)
    bad = {k: v for k, v in e.items() if not v <= TOL}
    assert not bad, bad


def test_fp8_backward_full_size():
    # the 2.7B shape, every element of every output against the oracle on the E4M3 values
    shape = inputs.workload("mamba2_2p7b").replace(dtype="fp8")
    print(f"[fp8 bwd full] {shape}", flush=True)
    inp = inputs.generate(shape, seed=34)
    got = run_fwd_bwd_gpu(inp, shape.chunk)
    ref = oracle_fwd_bwd(inp)
    e = {k: max_rel(got[k], ref[k]) for k in ref}
    print("  " + " ".join(f"{k}={v:.1e}" for k, v in e.items()), flush=True)
    bad = {k: v for k, v in e.items() if not v <= TOL}
    assert not bad, bad
