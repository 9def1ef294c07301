"""What FP8 (E4M3) x, B, C cost in accuracy, on the float64 oracle (CPU).

The same seeded draws are rounded once to bf16 and once to E4M3 (3 mantissa
bits: relative rounding error up to 2^-4 per value); the oracle's forward and
backward on each show the error the coarser operands introduce by themselves,
before any kernel arithmetic.  Each tensor's max|y_fp8 - y_bf16| / max|y_bf16| is printed;
the bound asserted is the loose one that documents the study, not a parity
tolerance (the library's FP8 path is checked against the oracle on the E4M3
values themselves, tests/test_gpu_fp8.py).
"""
import numpy as np
import pytest

from oracle import seq
from state_space_model_mamba2_amd import inputs
from tests.util import max_rel


def _fwd(inp):
    f = {k: inp.as_f64(k) for k in ("x", "dt", "A", "B", "C", "D")}
    return seq.ssd_fwd(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"])


@pytest.mark.parametrize("name,kw", [
    ("mamba2_370m", dict(batch=1, seqlen=512, nheads=4)),
    ("mamba2_2p7b", dict(batch=1, seqlen=1024, nheads=8)),
    ("zamba2_7b", dict(batch=1, seqlen=512, nheads=4, ngroups=2)),
    ("long_context", dict(batch=1, seqlen=1024, nheads=8, ngroups=2)),
])
def test_fp8_operand_error(name, kw):
    shape = inputs.workload(name, **kw)
    y16, f16 = _fwd(inputs.generate(shape.replace(dtype="bf16"), seed=40))
    y8, f8 = _fwd(inputs.generate(shape.replace(dtype="fp8"), seed=40))
    ey, ef = max_rel(y8, y16), max_rel(f8, f16)
    rms = float(np.sqrt(np.mean((y8 - y16) ** 2)) / np.sqrt(np.mean(y16 ** 2)))
    print(f"[fp8 study] {name}: y max-rel {ey:.3e} (rms rel {rms:.3e}), final_state {ef:.3e}")
    assert ey < 0.1 and ef < 0.1 and rms < 0.05


def _grads(inp):
    f = {k: inp.as_f64(k) for k in ("x", "dt", "A", "B", "C", "D", "dy")}
    g = seq.ssd_bwd(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["dy"])
    g.pop("dinitial_state")
    return g


@pytest.mark.parametrize("name,kw", [
    ("mamba2_370m", dict(batch=1, seqlen=512, nheads=4)),
    ("mamba2_2p7b", dict(batch=1, seqlen=1024, nheads=8)),
    ("zamba2_7b", dict(batch=1, seqlen=512, nheads=4, ngroups=2)),
    ("long_context", dict(batch=1, seqlen=1024, nheads=8, ngroups=2)),
])
def test_fp8_operand_error_backward(name, kw):
    # the gradients of the same loss <dy, y> with x, B, C rounded to E4M3
    # instead of bf16 (dy stays bf16 in both): the backward's share of the study
    shape = inputs.workload(name, **kw)
    g16 = _grads(inputs.generate(shape.replace(dtype="bf16"), seed=41))
    g8 = _grads(inputs.generate(shape.replace(dtype="fp8"), seed=41))
    e = {k: max_rel(g8[k], g16[k]) for k in g16}
    print(f"[fp8 study, backward] {name}: " + " ".join(f"{k}={v:.3e}" for k, v in e.items()))
    # dA sums dt_j dl_j over every token, and the per-token terms cancel to a
    # result far smaller than they are: on one head of the 370M-shape draw the
    # exact gradient is -4.9 with float32 operands, -6.3 with bf16 and +19.8
    # with E4M3.  It is reported, not bounded; every other gradient is.
    assert all(v < 0.1 for k, v in e.items() if k != "dA"), e
