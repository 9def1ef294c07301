"""Pins for the step-size preprocessing dt = softplus(dt_raw + dt_bias) (CPU only).

* softplus at points where it is known exactly or asymptotically, and as the
  inverse of the generator's inverse softplus ln(expm1(u));
* sigmoid as the finite-difference derivative of softplus, and the identity
  sigmoid(z) = 1 - exp(-softplus(z)) that lets a backward form the sigmoid
  from the stored step alone;
* central finite differences of <dy, y> + <dS_fin, final_state>, with the
  scan run on softplus(dt_raw + dt_bias), w.r.t. dt_raw and dt_bias.
"""
import math

import numpy as np

from oracle import dtproc, fd, seq
from tests.test_oracle import rand_inputs


def test_softplus_known_values():
    assert dtproc.softplus(0.0) == math.log(2.0)
    assert abs(dtproc.softplus(50.0) - 50.0) < 1e-15 * 50
    assert abs(dtproc.softplus(-50.0) - math.exp(-50.0)) < 1e-30
    assert abs(dtproc.softplus(1.0) - math.log(1.0 + math.e)) < 1e-15
    u = np.exp(np.linspace(math.log(1e-4), math.log(1e-1), 25))
    assert np.max(np.abs(dtproc.softplus(np.log(np.expm1(u))) - u) / u) < 1e-12


def test_sigmoid_is_the_derivative_and_matches_the_stored_step_form():
    z = np.linspace(-30.0, 30.0, 121)
    h = 1e-6
    num = (dtproc.softplus(z + h) - dtproc.softplus(z - h)) / (2 * h)
    assert np.max(np.abs(num - dtproc.sigmoid(z))) < 1e-8
    assert np.max(np.abs(-np.expm1(-dtproc.softplus(z)) - dtproc.sigmoid(z))) < 1e-15
    assert dtproc.sigmoid(0.0) == 0.5


def test_finite_differences_through_the_step():
    b, L, H, P, N, G = 2, 10, 4, 3, 5, 2
    inp, dy = rand_inputs(50, b, L, H, P, N, G)
    rng = np.random.default_rng(51)
    raw = rng.normal(0.0, math.sqrt(0.5), (b, L, H))
    bias = np.log(np.expm1(np.exp(rng.uniform(math.log(1e-3), math.log(1e-1), H))))
    dfs = rng.standard_normal((b, H, P, N))
    rest = {k: inp[k] for k in ("x", "A", "B", "C", "D")}

    def run(dt_raw, dt_bias):
        dt = dtproc.step(dt_raw, dt_bias)
        y, fs = seq.ssd_fwd(rest["x"], dt, rest["A"], rest["B"], rest["C"], rest["D"])
        return np.concatenate([y.ravel(), fs.ravel()])

    g = seq.ssd_bwd(rest["x"], dtproc.step(raw, bias), rest["A"], rest["B"], rest["C"], rest["D"], dy,
                    dfinal_state=dfs)
    ddt_raw, ddt_bias = dtproc.step_grads(g["ddt"], raw, bias)
    cot = np.concatenate([dy.ravel(), dfs.ravel()])
    vals = dict(dt_raw=raw, dt_bias=bias)
    for _ in range(8):
        idx = tuple(int(rng.integers(0, s)) for s in raw.shape)
        num = fd.central_diff(run, vals, "dt_raw", idx, cot, eps=1e-6)
        assert abs(num - ddt_raw[idx]) / max(1.0, np.abs(ddt_raw).max()) < 1e-7, (idx, num, ddt_raw[idx])
    for h in range(H):
        num = fd.central_diff(run, vals, "dt_bias", (h,), cot, eps=1e-6)
        assert abs(num - ddt_bias[h]) / max(1.0, np.abs(ddt_bias).max()) < 1e-7, (h, num, ddt_bias[h])


def test_no_bias_is_zero_bias():
    raw = np.random.default_rng(52).normal(size=(1, 5, 3))
    assert np.array_equal(dtproc.step(raw, None), dtproc.step(raw, np.zeros(3)))
    ddt = np.ones((1, 5, 3))
    a, ab = dtproc.step_grads(ddt, raw, None)
    b, bb = dtproc.step_grads(ddt, raw, np.zeros(3))
    assert np.array_equal(a, b) and np.array_equal(ab, bb)
