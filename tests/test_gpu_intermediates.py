"""Each kernel's own output against the float64 chunked oracle's intermediate.

The end-to-end parity tests see only y and the gradients; here the arrays the
kernels hand to one another are read back from the workspaces (their places
come from ssd_workspace_regions) after ssd_fwd and ssd_bwd, and compared with
the intermediates of oracle/chunked.py on the same seeded inputs:

  chunk cumsum          cs, the step dt           (float32 in every mode)
  chunk state           S_k                        (forward scratch)
  state passing         Hin_k, the state entering chunk k   (saved workspace)
  chunk state, reverse  dHloc_k                    (backward scratch)
  state passing, rev.   G_k = dH_{k+1}             (backward scratch)

States are compared chunk by chunk, each chunk's error over the largest value
of that chunk, so that a wrong chunk index shows even where the states are
small.  Tolerances: the float32 cumsum and step within 1e-5 of the largest
value; states as the outputs, 1e-4 with float32 storage and 2e-2 with bf16
storage (FP8 x, B, C against the oracle on the E4M3 values).  A shorter last
chunk is compared with the oracle's tail chunk; on its padded rows the step
must be 0 and the cumsum must hold the chunk's total.
"""
import ctypes

import numpy as np
import pytest

from state_space_model_mamba2_amd import inputs
from tests.util import NAMES_IN, max_rel

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 2e-2}
TOL_SCALAR = 1e-5


def _region(ws, off, count, dtype):
    esz = torch.tensor([], dtype=dtype).element_size()
    return ws[off:off + count * esz].view(dtype).float().cpu().numpy().astype(np.float64)


def run_gpu_intermediates(inp, chunk, states=None, softplus=False):
    from state_space_model_mamba2_amd import _lib, ssd

    dev = ssd.to_device(inp, "cuda")
    s0 = dfs = None
    if states is not None:
        s0, dfs = (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda() for a in states)
    dt = dev["dt_raw"] if softplus else dev["dt"]
    x, B = dev["x"], dev["B"]
    shape = ssd.shape_of(x, B, chunk, ssd._DTYPES[x.dtype], _lib.SSD_DT_SOFTPLUS if softplus else 0)
    lib = _lib.load()
    fscr = torch.zeros(lib.ssd_fwd_scratch_bytes(ctypes.byref(shape)), dtype=torch.uint8, device="cuda")
    bscr = torch.zeros(lib.ssd_bwd_scratch_bytes(ctypes.byref(shape)), dtype=torch.uint8, device="cuda")
    _, _, ctx = ssd.fwd(x, dt, dev["A"], B, dev["C"], dev["D"], chunk, initial_state=s0, dt_softplus=softplus,
                        dt_bias=dev["dt_bias"] if softplus else None, scratch=fscr)
    ssd.bwd(dev["dy"], ctx, dfinal_state=dfs, want_dinitial_state=states is not None, scratch=bscr)
    torch.cuda.synchronize()
    r = _lib.Regions()
    assert lib.ssd_workspace_regions(ctypes.byref(shape), ctypes.byref(r)) == _lib.SSD_OK
    b, L, H, P, N, Q = shape.batch, shape.seqlen, shape.nheads, shape.headdim, shape.dstate, shape.chunk
    K = -(-L // Q)
    sdt = torch.float32 if inp.shape.dtype == "f32" else torch.bfloat16
    nst = b * K * H * P * N
    return dict(
        cs=_region(ctx.saved_ws, r.cs, b * H * K * Q, torch.float32).reshape(b, H, K, Q),
        step=_region(ctx.saved_ws, r.step, b * H * K * Q, torch.float32).reshape(b, H, K, Q),
        Hin=_region(ctx.saved_ws, r.hin, nst, sdt).reshape(b, K, H, P, N),
        S=_region(fscr, r.chunk_state, nst, sdt).reshape(b, K, H, P, N),
        dHloc=_region(bscr, r.dhloc, nst, sdt).reshape(b, K, H, P, N),
        Gk=_region(bscr, r.gstate, nst, sdt).reshape(b, K, H, P, N),
    )


def run_oracle_intermediates(inp, chunk, states=None, softplus=False):
    from oracle import chunked, dtproc

    f = {k: inp.as_f64(k) for k in NAMES_IN + ["dy", "dt_raw", "dt_bias"]}
    dt = dtproc.step(f["dt_raw"], f["dt_bias"]) if softplus else f["dt"]
    s0, dfs = (None, None) if states is None else (np.asarray(a, np.float64) for a in states)
    out = chunked.ssd_chunked(f["x"], dt, f["A"], f["B"], f["C"], f["D"], chunk, dy=f["dy"], initial_state=s0,
                              dfinal_state=dfs)
    parts = [out["full"], out["tail"]] if "tail" in out else [out]
    b, L, H = dt.shape
    dts = [dt[:, :parts[0]["cs"].shape[1] * chunk]] + ([dt[:, (L // chunk) * chunk:]] if len(parts) > 1 else [])
    for p, d in zip(parts, dts):
        K, Qp = p["cs"].shape[1], p["cs"].shape[2]
        p["step"] = d.reshape(b, K, Qp, H)
        p["Hin"] = p["Hin"][:, :K]
    return parts


def _per_chunk(got, ref):
    return max(max_rel(got[:, k], ref[:, k]) for k in range(ref.shape[1])) if ref.shape[1] else 0.0


def _compare(shape, seed=0, states=False, softplus=False):
    print(f"[intermediates] {shape} states={states} softplus={softplus}", flush=True)
    inp = inputs.generate(shape, seed=seed)
    st = inputs.generate_states(shape, seed=seed) if states else None
    got = run_gpu_intermediates(inp, shape.chunk, st, softplus)
    parts = run_oracle_intermediates(inp, shape.chunk, st, softplus)
    tol = TOL[shape.dtype]
    errs = {}
    k0 = 0
    for part, ref in zip(["full", "tail"], parts):
        K, Qp = ref["cs"].shape[1], ref["cs"].shape[2]
        ks = slice(k0, k0 + K)
        for name in ("cs", "step"):
            g = got[name][:, :, ks, :Qp]                        # [b][H][k][i]
            r = np.moveaxis(ref[name], 3, 1)                    # [b][k][i][H] -> [b][H][k][i]
            errs[f"{part}.{name}"] = (max_rel(g, r), TOL_SCALAR)
        for name in ("S", "Hin", "dHloc", "Gk"):
            errs[f"{part}.{name}"] = (_per_chunk(got[name][:, ks], ref[name]), tol)
        if Qp < shape.chunk:                                    # zero-padded rows of a shorter last chunk
            step_t = got["step"][:, :, ks, Qp:]
            assert (step_t == 0).all(), "padded rows must have step 0"
            # the cumsum stays at the chunk's total (its last row is the
            # chunk's decay in the state kernels); it comes from the wave
            # scan's inclusive total, so it matches the last valid row up to
            # rounding, not bit for bit
            r_last = np.moveaxis(ref["cs"], 3, 1)[..., Qp - 1:Qp]
            errs[f"{part}.cs_pad"] = (max_rel(got["cs"][:, :, ks, Qp:], np.broadcast_to(r_last, step_t.shape)),
                                      TOL_SCALAR)
        k0 += K
    print("  " + " ".join(f"{k}={v:.2e}" for k, (v, _) in errs.items()), flush=True)
    bad = {k: v for k, (v, t) in errs.items() if not v <= t}
    assert not bad, f"{shape}: over tolerance: {bad}"


CASES = [
    (inputs.workload("tiny_fp32"), {}),
    (inputs.workload("tiny_fp32", chunk=128, seqlen=512, batch=2, nheads=4, ngroups=2), dict(states=True)),
    (inputs.workload("mamba2_370m", batch=2, seqlen=1024, nheads=4, chunk=64, dtype="f32"), {}),
    (inputs.workload("mamba2_370m", batch=2, seqlen=1024, nheads=4), {}),
    (inputs.workload("mamba2_370m", batch=2, seqlen=1024, nheads=4), dict(states=True, softplus=True)),
    (inputs.workload("zamba2_7b", batch=1, seqlen=768, nheads=8, ngroups=2), dict(states=True)),
    (inputs.workload("mamba2_2p7b", batch=1, seqlen=1024, nheads=4, ngroups=2, chunk=128), {}),
    (inputs.workload("mamba2_370m", batch=2, seqlen=1024, nheads=4, dtype="fp8"), dict(states=True)),
    # shorter last chunks: 900 = 3 x 256 + 132, 300 = 4 x 64 + 44, 100 < one chunk
    (inputs.workload("mamba2_370m", batch=2, seqlen=900, nheads=4), dict(states=True)),
    (inputs.workload("tiny_fp32", seqlen=300, batch=2, nheads=4, ngroups=2), dict(softplus=True)),
    (inputs.workload("mamba2_370m", batch=1, seqlen=100, nheads=4), {}),
]


@pytest.mark.parametrize("shape,kw", CASES,
                         ids=[f"{s.dtype}-L{s.seqlen}-Q{s.chunk}-H{s.nheads}-G{s.ngroups}-{'-'.join(kw) or 'plain'}"
                              for s, kw in CASES])
def test_kernel_intermediates(shape, kw):
    _compare(shape, seed=11, **kw)
