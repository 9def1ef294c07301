"""The chunk scans resident over heads (forward, and backward at chunk 256
with dstate a multiple of 64), on the shapes that reach their edge paths,
against the float64 oracle on every output.

The kernels take a (b, k, g) item and a slice of its heads per workgroup
when a slice holds at least 10 heads (the backward from 8; bf16 or FP8,
headdim 64).  Slices
are planned as about 256 workgroups: s = ceil(256 / items) slices of
per = ceil(heads per group / s) heads (at most 64), so the last slice may
hold fewer.  The shapes below are chosen to land on:

  * an odd head count per slice (the head loop's unpaired last step) and a
    shorter last chunk: 1 x (256 x 128 + 77) tokens, 11 heads, chunk 128
    -> 257 items, one slice of 11 heads (forward only), and the same at
    chunk 256: 1 x (256 x 256 + 77) tokens -> 257 items (both scans);
  * a shorter last slice: 4 x 4096 tokens, 42 heads, chunk 256 -> 64 items,
    slices of 11, 11, 11 and 9 heads (also with FP8 x, B, C, and with an
    initial state and a final-state cotangent);
  * dstate 64 and two groups: 1 x 16384 tokens, 40 heads in 2 groups ->
    128 items, two slices of 10 heads.

The full-size workload tests reach the same kernels with 20, 14 and 10
heads per slice, and the backward one also with 8 (Mamba2-370M shape).  Tolerance 2e-2 (max|gpu - oracle| / max|oracle|, bf16
storage; FP8 against the oracle on the E4M3 values).
"""
import os

import pytest

from state_space_model_mamba2_amd import inputs
from tests.util import max_rel, run_gpu, run_oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2


def _threads():
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    return min(n, int(omp)) if omp and omp.isdigit() and int(omp) > 0 else n


def _slice_plan(shape):
    # the slice arithmetic of the library's launch, restated to show which
    # path each case is meant to reach
    items = shape.batch * (-(-shape.seqlen // shape.chunk)) * shape.ngroups
    hpg = shape.nheads // shape.ngroups
    s = min(-(-256 // items), hpg)
    per = min(-(-hpg // s), 64)
    return per, -(-hpg // per)


CASES = [
    ("odd_heads_ragged", inputs.workload("mamba2_370m", batch=1, seqlen=256 * 128 + 77, nheads=11, chunk=128),
     dict(), (11, 1)),
    ("odd_heads_ragged_q256", inputs.workload("mamba2_370m", batch=1, seqlen=256 * 256 + 77, nheads=11, chunk=256),
     dict(), (11, 1)),
    ("short_last_slice", inputs.workload("mamba2_2p7b", batch=4, seqlen=4096, nheads=42), dict(), (11, 4)),
    ("short_last_slice_fp8", inputs.workload("mamba2_2p7b", batch=4, seqlen=4096, nheads=42, dtype="fp8"),
     dict(), (11, 4)),
    ("short_last_slice_states", inputs.workload("mamba2_2p7b", batch=4, seqlen=4096, nheads=42),
     dict(states=True), (11, 4)),
    ("dstate64_two_groups", inputs.workload("zamba2_7b", batch=1, seqlen=16384, nheads=40, ngroups=2),
     dict(), (10, 2)),
]


@pytest.mark.parametrize("name,shape,kw,plan", CASES, ids=[c[0] for c in CASES])
def test_resident_forward_scan(name, shape, kw, plan):
    assert _slice_plan(shape) == plan
    print(f"[resident] {name}: {shape} heads per slice, slices = {plan}", flush=True)
    inp = inputs.generate(shape, seed=17)
    states = inputs.generate_states(shape, seed=17) if kw.get("states") else None
    got, _ = run_gpu(inp, shape.chunk, states=states)
    ref = run_oracle(inp, nthreads=_threads(), states=states)
    errs = {k: max_rel(got[k], ref[k]) for k in ref}
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, f"{name}: over tolerance {TOL}: {bad}"
