"""libssd on sequences whose length is not a multiple of the chunk length.

The whole chunks run in place; the remaining tokens of every sequence run as
one zero-padded chunk that starts from the state the whole chunks leave.  The
oracle is the sequential recurrence, which has no chunks at all, so parity
checks the tail handling directly.  Tolerance as elsewhere: per tensor
max|gpu - oracle| / max|oracle| <= 1e-4 (fp32) or 2e-2 (bf16).
"""
import numpy as np
import pytest

from state_space_model_mamba2_amd import inputs
from tests.util import max_rel, run_gpu, run_oracle, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}

CASES = [
    # (workload, overrides): remainders 1, 37, Q - 24, Q - 1 and sequences shorter than one chunk
    ("tiny_fp32", dict(batch=2, seqlen=64 * 3 + 1, nheads=4, ngroups=2)),
    ("tiny_fp32", dict(batch=2, seqlen=50, nheads=4, ngroups=2)),
    ("mamba2_370m", dict(batch=2, seqlen=64 * 4 + 37, nheads=4, chunk=64, dtype="f32")),
    ("mamba2_370m", dict(batch=2, seqlen=1000, nheads=4)),
    ("mamba2_370m", dict(batch=2, seqlen=255, nheads=4)),
    ("mamba2_370m", dict(batch=3, seqlen=128 * 3 + 1, nheads=4, ngroups=2, chunk=128)),
    ("zamba2_7b", dict(batch=1, seqlen=700, nheads=8, ngroups=2)),
    ("tiny_fp32", dict(batch=2, seqlen=77, nheads=2, chunk=128, dtype="bf16")),
]


def _id(case):
    name, kw = case
    s = inputs.workload(name, **kw)
    return f"{s.dtype}-Q{s.chunk}-P{s.headdim}-N{s.dstate}-G{s.ngroups}-L{s.seqlen}"


def _compare(got, ref, tol, what):
    assert set(got) == set(ref)
    errs = {k: max_rel(got[k], ref[k]) for k in ref}
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{what}: over tolerance {tol}: {bad}"


@pytest.mark.parametrize("with_states", [False, True])
@pytest.mark.parametrize("case", CASES, ids=_id)
def test_ragged_parity(case, with_states):
    name, kw = case
    shape = inputs.workload(name, **kw)
    print(f"[ragged] {shape} states={with_states}", flush=True)
    inp = inputs.generate(shape, seed=7)
    st = inputs.generate_states(shape, seed=7) if with_states else None
    got, _ = run_gpu(inp, shape.chunk, states=st)
    ref = run_oracle(inp, states=st)
    _compare(got, ref, TOL[shape.dtype], shape)


def test_ragged_is_deterministic():
    shape = inputs.workload("mamba2_370m", batch=2, seqlen=777, nheads=4)
    print(f"[ragged determinism] {shape}", flush=True)
    inp = inputs.generate(shape, seed=8)
    st = inputs.generate_states(shape, seed=8)
    a, _ = run_gpu(inp, shape.chunk, states=st)
    b, _ = run_gpu(inp, shape.chunk, states=st)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_full_size_ragged_sampled_parity():
    """The 2.7B workload shortened to 4000 tokens (15 whole chunks and 160
    tokens): batch row 0, every head, against the oracle."""
    import os

    from oracle import seq

    shape = inputs.workload("mamba2_2p7b", seqlen=4000)
    print(f"[ragged full] {shape}", flush=True)
    inp = inputs.generate(shape, seed=9)
    got, _ = run_gpu(inp, shape.chunk)
    sub = {k: inp.as_f64(k)[:1] for k in ("x", "dt", "B", "C", "dy")}
    nt = min(len(os.sched_getaffinity(0)), 16)
    A, D = inp.as_f64("A"), inp.as_f64("D")
    ry, rfs = seq.ssd_fwd(sub["x"], sub["dt"], A, sub["B"], sub["C"], D, nthreads=nt)
    rg = seq.ssd_bwd(sub["x"], sub["dt"], A, sub["B"], sub["C"], D, sub["dy"], nthreads=nt)
    keys = ("dx", "ddt", "dB", "dC")
    ref = dict(y=ry, final_state=rfs, **{k: rg[k] for k in keys})
    mine = dict(y=got["y"][:1], final_state=got["final_state"][:1], **{k: got[k][:1] for k in keys})
    _compare(mine, ref, TOL["bf16"], shape)


def test_uneven_cut_of_long_context():
    """The long-context workload cut at token 30001 (neither piece a multiple
    of the chunk) and run as two chained calls agrees with the one-call run."""
    from state_space_model_mamba2_amd import ssd

    shape = inputs.workload("long_context")
    print(f"[ragged cut] {shape}", flush=True)
    inp = inputs.generate(shape, seed=10)
    dev = ssd.to_device(inp, "cuda")
    y, fs, ctx = ssd.fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], shape.chunk)
    g = ssd.bwd(dev["dy"], ctx)
    torch.cuda.synchronize()
    whole = dict(y=to_np(y), final_state=to_np(fs), **{k: to_np(v) for k, v in g.items()})
    del y, fs, ctx, g
    cut = 30001

    def part(name, lo, hi):
        return dev[name][:, lo:hi].contiguous()

    y1, f1, c1 = ssd.fwd(part("x", 0, cut), part("dt", 0, cut), dev["A"], part("B", 0, cut), part("C", 0, cut),
                         dev["D"], shape.chunk)
    L = shape.seqlen
    y2, f2, c2 = ssd.fwd(part("x", cut, L), part("dt", cut, L), dev["A"], part("B", cut, L), part("C", cut, L),
                         dev["D"], shape.chunk, initial_state=f1)
    g2 = ssd.bwd(part("dy", cut, L), c2, want_dinitial_state=True)
    g1 = ssd.bwd(part("dy", 0, cut), c1, dfinal_state=g2["dinitial_state"])
    torch.cuda.synchronize()
    split = dict(y=to_np(torch.cat([y1, y2], 1)), final_state=to_np(f2))
    for k in ("dx", "ddt", "dB", "dC"):
        split[k] = to_np(torch.cat([g1[k], g2[k]], 1))
    for k in ("dA", "dD"):
        split[k] = to_np(g1[k].double() + g2[k].double())
    _compare(split, whole, TOL["bf16"], "uneven cut")
