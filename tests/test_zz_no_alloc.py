"""ssd_fwd_noalloc (the forward whose scratch is the library's static device
buffer) against ssd_fwd, called through the C ABI on the GPU: two calls in
a row, the second on a smaller problem with a shorter last chunk, each
compared element by element with ssd_fwd on the same inputs.  Both run the
same kernels on the same inputs, so y and final_state must agree bit for
bit, and the backward from the context ssd_fwd_noalloc filled must give the
gradients of the backward from ssd_fwd's context."""
import ctypes

import numpy as np
import pytest

from state_space_model_mamba2_amd import _lib, inputs
from tests.util import max_rel, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = [
    # (workload, overrides, with initial state)
    ("mamba2_370m", dict(batch=2, seqlen=2048), True),
    ("mamba2_2p7b", dict(batch=1, seqlen=1000, nheads=8, ngroups=2), False),
]


def _noalloc_fwd(dev, shape_obj, s0):
    lib = _lib.load()
    x, dt, A, B, C, D = (dev[k] for k in ("x", "dt", "A", "B", "C", "D"))
    saved_bytes = lib.ssd_saved_bytes(ctypes.byref(shape_obj))
    assert lib.ssd_fwd_scratch_bytes(ctypes.byref(shape_obj)) <= _lib.SSD_FWD_STATIC_SCRATCH_BYTES
    y = torch.empty_like(x)
    fs = torch.empty((shape_obj.batch, shape_obj.nheads, shape_obj.headdim, shape_obj.dstate),
                     dtype=torch.float32, device=x.device)
    saved_ws = torch.empty(saved_bytes, dtype=torch.uint8, device=x.device)
    saved = _lib.Saved()
    code = lib.ssd_fwd_noalloc(ctypes.byref(shape_obj), x.data_ptr(), dt.data_ptr(), A.data_ptr(), B.data_ptr(),
                               C.data_ptr(), D.data_ptr(), None, s0.data_ptr() if s0 is not None else None,
                               y.data_ptr(), fs.data_ptr(), saved_ws.data_ptr(), saved_bytes, ctypes.byref(saved),
                               torch.cuda.current_stream().cuda_stream, None)
    assert code == _lib.SSD_OK, _lib.status_string(code)
    return y, fs, saved, saved_ws


def test_noalloc_forward_matches_ssd_fwd_twice():
    from state_space_model_mamba2_amd import ssd

    for name, over, with_state in CASES:
        shape = inputs.workload(name, **over)
        print(f"[noalloc] {name} {over}: {shape}", flush=True)
        inp = inputs.generate(shape, seed=0)
        dev = ssd.to_device(inp, "cuda")
        s0 = None
        if with_state:
            s0 = torch.from_numpy(inputs.generate_states(shape, seed=0)[0]).cuda()
        y_ref, fs_ref, ctx = ssd.fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], shape.chunk,
                                     initial_state=s0)
        g_ref = ssd.bwd(dev["dy"], ctx)
        y, fs, saved, saved_ws = _noalloc_fwd(dev, ctx.shape, s0)
        # the backward from the no-allocation forward's context (its saved workspace is the caller's)
        ctx2 = ssd.Context(saved, ctx.tensors, saved_ws, ctx.shape, ctx.dtype)
        g = ssd.bwd(dev["dy"], ctx2)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), "y differs from ssd_fwd"
        assert torch.equal(fs, fs_ref), "final_state differs from ssd_fwd"
        errs = {k: max_rel(to_np(g[k]), to_np(g_ref[k])) for k in g_ref}
        print("  grads vs ssd_fwd's context: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
        for k in g_ref:
            assert torch.equal(g[k].view(torch.uint8) if g[k].dtype != torch.float32 else g[k],
                               g_ref[k].view(torch.uint8) if g_ref[k].dtype != torch.float32 else g_ref[k]), k
        assert np.isfinite(to_np(y)).all()
