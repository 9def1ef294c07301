"""Parity of libssd (HIP, gfx950) against the float64 oracle on seeded inputs.

Tolerance: per tensor, max|gpu - oracle| / max|oracle| <= 1e-4 for fp32
storage and <= 2e-2 for bf16 storage with fp32 accumulation.
"""
import numpy as np
import pytest

from state_space_model_mamba2_amd import inputs
from tests.util import GRADS, max_rel, run_gpu, run_oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _check(shape, seed=0, tol=None):
    print(f"[parity] {shape}", flush=True)
    inp = inputs.generate(shape, seed=seed)
    got, _ = run_gpu(inp, shape.chunk)
    ref = run_oracle(inp)
    tol = TOL[shape.dtype] if tol is None else tol
    errs = {k: max_rel(got[k], ref[k]) for k in ref}
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{shape}: over tolerance {tol}: {bad}"
    return errs


def test_tiny_fp32_workload():
    _check(inputs.workload("tiny_fp32"))


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_tiny_shape_chunks_fp32(chunk):
    _check(inputs.workload("tiny_fp32", chunk=chunk, seqlen=512, batch=2, nheads=4, ngroups=2))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mamba2_head_shape_small(dtype):
    # headdim 64, dstate 128 as in the 370M / 2.7B workloads, few heads and tokens
    chunk = 256 if dtype == "bf16" else 64
    _check(inputs.workload("mamba2_370m", batch=2, seqlen=1024, nheads=4, chunk=chunk, dtype=dtype))


def test_zamba_head_shape_small():
    _check(inputs.workload("zamba2_7b", batch=1, seqlen=768, nheads=8, ngroups=2))


# The chunk-64 case faulted the GPU once under an 8-wave rewrite of the
# backward chunk kernel (since withdrawn); no cause was found in that code's
# source or ISA, so the case stays off the GPU until one is shown, and the
# library reports bf16 at chunk 64 as unsupported.
FAULTED_UNEXPLAINED = ("GPU memory fault under a withdrawn 8-wave backward chunk kernel; cause not yet identified "
                       "(bf16 chunk 64 is switched off in the library)")


@pytest.mark.parametrize("chunk", [pytest.param(64, marks=pytest.mark.skip(reason=FAULTED_UNEXPLAINED)), 128])
def test_bf16_smaller_chunks(chunk):
    _check(inputs.workload("mamba2_2p7b", batch=1, seqlen=1024, nheads=4, ngroups=2, chunk=chunk))


def test_long_context_decay_small():
    _check(inputs.workload("long_context", seqlen=2048, nheads=8, ngroups=4))


# The remaining compiled bf16 (chunk, headdim, dstate) combinations.
@pytest.mark.parametrize("chunk,headdim,dstate", [(128, 16, 16), (256, 16, 16), (128, 64, 64), (256, 64, 64)])
def test_bf16_other_configs(chunk, headdim, dstate):
    _check(inputs.workload("mamba2_370m", batch=2, seqlen=512, nheads=4, ngroups=2, chunk=chunk,
                           headdim=headdim, dstate=dstate))


# Head counts per group that do not split evenly into head slices (5, 6, 9
# heads; one chunk, so the group-level backward kernels ask for the most
# slices): every slice must hold at least one head.
@pytest.mark.parametrize("nheads,ngroups,dtype,chunk",
                         [(9, 1, "f32", 64), (10, 2, "f32", 64), (6, 1, "bf16", 128), (9, 1, "bf16", 256)])
def test_uneven_head_slices(nheads, ngroups, dtype, chunk):
    _check(inputs.workload("tiny_fp32", batch=1, seqlen=chunk, nheads=nheads, ngroups=ngroups, chunk=chunk,
                           dtype=dtype))


# Launch shapes whose work-item counts fit no launch granularity: 3 x 700
# tokens (a shorter last chunk) with 10 heads in 2 groups gives 90 (b, k, h)
# items (the XCD-aware item map pads to 96), an odd head count per group (one
# head per chunk-state workgroup) and a last dl-assembly workgroup with 2 of
# its 4 head waves.  8192 tokens in 8 groups give 256 (b, k, g) items, enough
# for the dC/dB finalisation to take all dstate columns in one workgroup.
@pytest.mark.parametrize("shape", [
    dict(base="mamba2_370m", batch=3, seqlen=700, nheads=10, ngroups=2),
    dict(base="long_context", batch=1, seqlen=8192, nheads=8, ngroups=8),
], ids=["ragged_10_heads_2_groups", "8_groups_8192_tokens"])
def test_launch_shape_edges(shape):
    shape = dict(shape)
    _check(inputs.workload(shape.pop("base"), **shape))
