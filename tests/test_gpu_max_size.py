"""The largest shapes: element offsets past 2^31.

Eight batch rows of the long-context workload (8 x 65536 tokens, 80 heads,
headdim 64, dstate 128, 8 groups, chunk 256, bf16).  x, dy, y and dx hold
2.7e9 elements each, so the last batch rows sit past 2^31 elements, and the
per-chunk state buffers and the dW head-slice partials past 2^31 bytes.

Input recipe: to keep generation small, batch row b is the seeded one-row
long-context draw rotated in time by b * 4099 tokens (x, dt, B, C and dy
rotated together), so every row is a different sequence and a kernel that
mixed up batch rows would read the wrong one.  The float64 oracle computes
sampled outputs exactly:
  * batch row 7, every head of group 7: y, final_state, dx, ddt, dB, dC;
  * heads 78 and 79 over all eight rows: dA, dD (sums over batch and tokens).
Tolerance: max|gpu - oracle| / max|oracle| <= 2e-2 per tensor (bf16 storage,
fp32 accumulation).
"""
import os

import numpy as np
import pytest

from state_space_model_mamba2_amd import inputs
from tests.util import max_rel, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2
ROWS = 8
SHIFT = 4099


def _f64(a):
    a = np.ascontiguousarray(a)
    return (inputs.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def _threads():
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    return min(n, int(omp)) if omp and omp.isdigit() and int(omp) > 0 else n


def _row(a, b, sl):
    """Columns sl (heads or groups) of batch row b of a time-major [1][L][...]
    array: rotated in time by b * SHIFT tokens."""
    return np.roll(a[0][:, sl], b * SHIFT, axis=0)


@pytest.mark.timeout(900)
def test_offsets_past_2_to_the_31():
    from oracle import seq
    from state_space_model_mamba2_amd import ssd

    shape = inputs.workload("long_context")
    assert shape.batch == 1
    H, G, L = shape.nheads, shape.ngroups, shape.seqlen
    hg = H // G
    print(f"[max size] {ROWS} x long_context rows: {shape}", flush=True)
    inp = inputs.generate(shape, seed=0)
    d1 = ssd.to_device(inp, "cuda")
    big = {k: torch.cat([torch.roll(d1[k], b * SHIFT, dims=1) for b in range(ROWS)]).contiguous()
           for k in ("x", "dt", "B", "C", "dy")}
    assert big["x"].numel() > 2 ** 31
    A, D = d1["A"], d1["D"]
    del d1
    y, fs, ctx = ssd.fwd(big["x"], big["dt"], A, big["B"], big["C"], D, shape.chunk)
    g = ssd.bwd(big["dy"], ctx)
    torch.cuda.synchronize()
    print("[max size] GPU forward and backward done", flush=True)

    b, gl = ROWS - 1, G - 1
    hs = slice(gl * hg, (gl + 1) * hg)
    gs = slice(gl, gl + 1)
    o_in = dict(x=_f64(_row(inp.x, b, hs)[None]), dt=_f64(_row(inp.dt, b, hs)[None]), A=_f64(inp.A[hs]),
                B=_f64(_row(inp.B, b, gs)[None]), C=_f64(_row(inp.C, b, gs)[None]), D=_f64(inp.D[hs]))
    nt = _threads()
    ry, rfs = seq.ssd_fwd(**o_in, nthreads=nt)
    rg = seq.ssd_bwd(**o_in, dy=_f64(_row(inp.dy, b, hs)[None]), nthreads=nt)
    got = {
        "y": to_np(y[b:b + 1, :, hs]), "final_state": to_np(fs[b:b + 1, hs]),
        "dx": to_np(g["dx"][b:b + 1, :, hs]), "ddt": to_np(g["ddt"][b:b + 1, :, hs]),
        "dB": to_np(g["dB"][b:b + 1, :, gl:gl + 1]), "dC": to_np(g["dC"][b:b + 1, :, gl:gl + 1]),
    }
    ref = {"y": ry, "final_state": rfs, "dx": rg["dx"], "ddt": rg["ddt"], "dB": rg["dB"], "dC": rg["dC"]}
    print("[max size] oracle sample 1 done", flush=True)

    h2 = slice(H - 2, H)
    stack = lambda a, sl: np.stack([_row(a, r, sl) for r in range(ROWS)])
    o2 = dict(x=_f64(stack(inp.x, h2)), dt=_f64(stack(inp.dt, h2)), A=_f64(inp.A[h2]),
              B=_f64(stack(inp.B, gs)), C=_f64(stack(inp.C, gs)), D=_f64(inp.D[h2]))
    rg2 = seq.ssd_bwd(**o2, dy=_f64(stack(inp.dy, h2)), nthreads=nt)
    got["dA"], ref["dA"] = to_np(g["dA"][h2]), rg2["dA"]
    got["dD"], ref["dD"] = to_np(g["dD"][h2]), rg2["dD"]

    errs = {k: max_rel(got[k], ref[k]) for k in ref}
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    del big, y, fs, ctx, g
    torch.cuda.empty_cache()
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, f"over tolerance {TOL}: {bad}"
