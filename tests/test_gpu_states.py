"""libssd with an initial state, a final-state cotangent and the initial-state
gradient, on the GPU.

* Parity with the float64 oracle on seeded inputs and seeded states, every
  output including dinitial_state (tolerance: 1e-4 fp32, 2e-2 bf16, as
  max|gpu - oracle| / max|oracle| per tensor).
* Passing all-zero states gives bitwise the same results as passing none.
* A sequence cut into consecutive pieces and run as chained calls (each
  forward starts from the previous final_state; each backward takes the next
  piece's dinitial_state as its dfinal_state) reproduces the one-call results
  at full size: the long-context workload in eight pieces of 8192 tokens (the
  per-GPU share of an eight-way sequence split) and the 2.7B workload in two.
"""
import numpy as np
import pytest

from state_space_model_mamba2_amd import inputs
from tests.util import max_rel, run_gpu, run_oracle, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}

SMALL = [
    inputs.workload("tiny_fp32"),
    inputs.workload("tiny_fp32", chunk=128, seqlen=512, batch=2, nheads=4, ngroups=2),
    inputs.workload("mamba2_370m", batch=2, seqlen=1024, nheads=4, chunk=64, dtype="f32"),
    inputs.workload("mamba2_370m", batch=2, seqlen=1024, nheads=4),
    inputs.workload("mamba2_370m", batch=2, seqlen=512, nheads=4, ngroups=2, chunk=128),
    inputs.workload("zamba2_7b", batch=1, seqlen=768, nheads=8, ngroups=2),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: f"{s.dtype}-Q{s.chunk}-P{s.headdim}-N{s.dstate}-G{s.ngroups}")
def test_states_parity(shape):
    print(f"[states] {shape}", flush=True)
    inp = inputs.generate(shape, seed=3)
    st = inputs.generate_states(shape, seed=3)
    got, _ = run_gpu(inp, shape.chunk, states=st)
    ref = run_oracle(inp, states=st)
    assert set(ref) == set(got)
    errs = {k: max_rel(got[k], ref[k]) for k in ref}
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    tol = TOL[shape.dtype]
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{shape}: over tolerance {tol}: {bad}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_states_equal_no_states(dtype):
    chunk = 64 if dtype == "f32" else 256
    shape = inputs.workload("mamba2_370m", batch=2, seqlen=512, nheads=4, chunk=chunk, dtype=dtype)
    print(f"[zero states] {shape}", flush=True)
    inp = inputs.generate(shape, seed=4)
    z = np.zeros((shape.batch, shape.nheads, shape.headdim, shape.dstate), np.float32)
    a, _ = run_gpu(inp, shape.chunk)
    b, _ = run_gpu(inp, shape.chunk, states=(z, z))
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    # the initial-state gradient does not depend on the initial state itself
    ref = run_oracle(inp, states=(z, z))["dinitial_state"]
    assert max_rel(b["dinitial_state"], ref) <= TOL[dtype]


def _run_pieces(dev, shape, bounds, s0, dfs):
    """Chained forward over the pieces, then chained backward in reverse."""
    from state_space_model_mamba2_amd import ssd

    def piece(name, lo, hi):
        return dev[name][:, lo:hi].contiguous()

    ctxs, ys = [], []
    state = s0
    for lo, hi in bounds:
        y, state, ctx = ssd.fwd(piece("x", lo, hi), piece("dt", lo, hi), dev["A"], piece("B", lo, hi),
                                piece("C", lo, hi), dev["D"], shape.chunk, initial_state=state)
        ctxs.append(ctx)
        ys.append(y)
    grads = [None] * len(bounds)
    cot = dfs
    for i in reversed(range(len(bounds))):
        lo, hi = bounds[i]
        g = ssd.bwd(piece("dy", lo, hi), ctxs[i], dfinal_state=cot, want_dinitial_state=True)
        cot = g["dinitial_state"]
        grads[i] = g
    torch.cuda.synchronize()
    out = dict(y=torch.cat(ys, 1), final_state=state, dinitial_state=cot)
    for k in ("dx", "ddt", "dB", "dC"):
        out[k] = torch.cat([g[k] for g in grads], 1)
    for k in ("dA", "dD"):
        out[k] = sum(g[k].double() for g in grads)
    return {k: to_np(v) for k, v in out.items()}


@pytest.mark.parametrize("name,pieces", [("long_context", 8), ("mamba2_2p7b", 2)])
def test_sequence_split_into_chained_calls(name, pieces):
    from state_space_model_mamba2_amd import ssd

    shape = inputs.workload(name)
    print(f"[split] {name} into {pieces} pieces", flush=True)
    inp = inputs.generate(shape, seed=5)
    s0, dfs = inputs.generate_states(shape, seed=5)
    dev = ssd.to_device(inp, "cuda")
    ts0 = torch.from_numpy(s0).cuda()
    tdfs = torch.from_numpy(dfs).cuda()
    y, fs, ctx = ssd.fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], shape.chunk, initial_state=ts0)
    g = ssd.bwd(dev["dy"], ctx, dfinal_state=tdfs, want_dinitial_state=True)
    torch.cuda.synchronize()
    whole = dict(y=to_np(y), final_state=to_np(fs), **{k: to_np(v) for k, v in g.items()})
    del y, fs, ctx, g
    L = shape.seqlen // pieces
    split = _run_pieces(dev, shape, [(i * L, (i + 1) * L) for i in range(pieces)], ts0, tdfs)
    errs = {k: max_rel(split[k], whole[k]) for k in whole}
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    # Both runs do the same per-chunk arithmetic and carry the state in fp32
    # across the cuts; they differ only in how the group-level head sums (dB,
    # dC: a different head slicing can flip the last bf16 bit) and the chunk
    # sums of dA / dD are split.
    for k in ("y", "final_state", "dx", "ddt", "dinitial_state"):
        assert errs[k] <= 1e-6, (k, errs[k])
    for k in ("dB", "dC"):
        assert errs[k] <= 1e-2, (k, errs[k])
    for k in ("dA", "dD"):
        assert errs[k] <= 1e-4, (k, errs[k])


def test_full_size_states_sampled_parity():
    """The 2.7B workload with states: batch row 0 and every head (one group)
    against the oracle."""
    import os

    from oracle import seq
    from state_space_model_mamba2_amd import ssd

    shape = inputs.workload("mamba2_2p7b")
    print(f"[states full] {shape}", flush=True)
    inp = inputs.generate(shape, seed=6)
    s0, dfs = inputs.generate_states(shape, seed=6)
    dev = ssd.to_device(inp, "cuda")
    y, fs, ctx = ssd.fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], shape.chunk,
                         initial_state=torch.from_numpy(s0).cuda())
    g = ssd.bwd(dev["dy"], ctx, dfinal_state=torch.from_numpy(dfs).cuda(), want_dinitial_state=True)
    torch.cuda.synchronize()
    sub = {k: inp.as_f64(k)[:1] for k in ("x", "dt", "B", "C", "dy")}
    nt = min(len(os.sched_getaffinity(0)), 16)
    ry, rfs = seq.ssd_fwd(sub["x"], sub["dt"], inp.as_f64("A"), sub["B"], sub["C"], inp.as_f64("D"),
                          initial_state=s0[:1].astype(np.float64), nthreads=nt)
    rg = seq.ssd_bwd(sub["x"], sub["dt"], inp.as_f64("A"), sub["B"], sub["C"], inp.as_f64("D"), sub["dy"],
                     initial_state=s0[:1].astype(np.float64), dfinal_state=dfs[:1].astype(np.float64), nthreads=nt)
    got = dict(y=to_np(y[:1]), final_state=to_np(fs[:1]), dinitial_state=to_np(g["dinitial_state"][:1]),
               dx=to_np(g["dx"][:1]), ddt=to_np(g["ddt"][:1]), dB=to_np(g["dB"][:1]), dC=to_np(g["dC"][:1]))
    ref = dict(y=ry, final_state=rfs, dinitial_state=rg["dinitial_state"], dx=rg["dx"], ddt=rg["ddt"],
               dB=rg["dB"], dC=rg["dC"])
    errs = {k: max_rel(got[k], ref[k]) for k in ref}
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
    assert not bad, bad
