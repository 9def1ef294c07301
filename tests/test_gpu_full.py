"""Full-size workloads on the GPU, in the launch configuration bench.py times.

The float64 oracle cannot run a whole workload in test time, so each
workload is checked on sampled outputs the oracle computes exactly:
  * batch row 0 and every head of group 0: y, final_state, dx, ddt, dB, dC
    (dB/dC of a group need all of its heads),
  * every batch row of two heads: dA and dD (sums over batch and tokens),
and on properties that hold at any size (the homogeneity identities, see
test_gpu_properties.py).  Tolerance: max|gpu - oracle| / max|oracle| <= 2e-2
over the sampled entries (bf16 storage, fp32 accumulation).
"""
import os

import numpy as np
import pytest

from state_space_model_mamba2_amd import inputs
from tests.util import max_rel, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2
WORKLOADS = ["mamba2_370m", "mamba2_2p7b", "zamba2_7b", "long_context"]


def _f64(a):
    a = np.ascontiguousarray(a)
    return (inputs.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def _threads():
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    return min(n, int(omp)) if omp and omp.isdigit() and int(omp) > 0 else n


@pytest.mark.parametrize("name", WORKLOADS)
def test_full_size_sampled_parity(name):
    from oracle import seq
    from state_space_model_mamba2_amd import ssd

    shape = inputs.workload(name)
    print(f"[full] {name}: {shape}", flush=True)
    inp = inputs.generate(shape, seed=0)
    dev = ssd.to_device(inp, "cuda")
    y, fs, ctx = ssd.fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], shape.chunk)
    g = ssd.bwd(dev["dy"], ctx)
    torch.cuda.synchronize()
    H, G = shape.nheads, shape.ngroups
    hg = H // G
    # sample 1: batch row 0, heads of group 0
    sl = (slice(0, 1), slice(None), slice(0, hg))
    o_in = dict(x=_f64(inp.x[sl]), dt=_f64(inp.dt[sl]), A=_f64(inp.A[:hg]), B=_f64(inp.B[:1, :, :1]),
                C=_f64(inp.C[:1, :, :1]), D=_f64(inp.D[:hg]))
    nt = _threads()
    ry, rfs = seq.ssd_fwd(**o_in, nthreads=nt)
    rg = seq.ssd_bwd(**o_in, dy=_f64(inp.dy[sl]), nthreads=nt)
    got = {
        "y": to_np(y[:1, :, :hg]), "final_state": to_np(fs[:1, :hg]),
        "dx": to_np(g["dx"][:1, :, :hg]), "ddt": to_np(g["ddt"][:1, :, :hg]),
        "dB": to_np(g["dB"][:1, :, :1]), "dC": to_np(g["dC"][:1, :, :1]),
    }
    ref = {"y": ry, "final_state": rfs, "dx": rg["dx"], "ddt": rg["ddt"], "dB": rg["dB"], "dC": rg["dC"]}
    # sample 2: all batch rows, two heads of group 0
    hs = slice(0, 2)
    o2 = dict(x=_f64(inp.x[:, :, hs]), dt=_f64(inp.dt[:, :, hs]), A=_f64(inp.A[hs]), B=_f64(inp.B[:, :, :1]),
              C=_f64(inp.C[:, :, :1]), D=_f64(inp.D[hs]))
    rg2 = seq.ssd_bwd(**o2, dy=_f64(inp.dy[:, :, hs]), nthreads=nt)
    got["dA"] = to_np(g["dA"][:2])
    got["dD"] = to_np(g["dD"][:2])
    ref["dA"] = rg2["dA"]
    ref["dD"] = rg2["dD"]
    errs = {k: max_rel(got[k], ref[k]) for k in ref}
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, f"{name}: over tolerance {TOL}: {bad}"
