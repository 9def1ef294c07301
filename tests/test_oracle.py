"""Pins for the float64 oracle (CPU only).

The pages print no formula and no worked example for the SSD scan, so the
oracle is pinned by things independent of its own code:
  * a three-step example worked by hand (tests/golden/hand_worked_L3.json),
  * the quadratic masked-attention (dual) form, an O(L^2) brute force,
  * central finite differences of <dy, y> for every gradient,
  * the chunked evaluation at every chunk length that divides L,
  * closed forms: L = 1, A = 0 (cumulative linear attention), a_t = 0
    (memoryless), N = P = 1 (a first-order IIR filter, scipy.signal.lfilter),
    B = 0 and x = 0,
  * exact homogeneity identities that any correct gradient satisfies.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal

from oracle import chunked, dual, fd, seq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(seed, b, L, H, P, N, G, a_max=4.0, dt_scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, L, H, P))
    dt = dt_scale * np.log1p(np.exp(rng.standard_normal((b, L, H))))
    A = -np.exp(rng.uniform(0.0, math.log(a_max), H))
    B = rng.standard_normal((b, L, G, N))
    C = rng.standard_normal((b, L, G, N))
    D = rng.standard_normal(H)
    dy = rng.standard_normal((b, L, H, P))
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D), dy


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / (den if den > 0 else 1.0))


SHAPES = [  # b, L, H, P, N, G
    (1, 1, 1, 1, 1, 1),
    (2, 12, 4, 3, 5, 2),
    (1, 17, 3, 2, 4, 1),
    (2, 9, 6, 4, 3, 3),
]


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_worked_L3.json")) as f:
        g = json.load(f)
    i, e = g["inputs"], g["expected"]
    sh = (1, 3, 1, 1)
    x = np.array(i["x"]).reshape(sh)
    dt = np.array(i["dt"]).reshape(1, 3, 1)
    A = np.array([-math.log(2.0)])
    B = np.array(i["B"]).reshape(1, 3, 1, 1)
    C = np.array(i["C"]).reshape(1, 3, 1, 1)
    D = np.array([i["D"]])
    dy = np.array(i["dy"]).reshape(sh)
    y, fs = seq.ssd_fwd(x, dt, A, B, C, D)
    np.testing.assert_allclose(y.ravel(), e["y"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(fs.ravel(), [e["final_state"]], rtol=0, atol=1e-14)
    gr = seq.ssd_bwd(x, dt, A, B, C, D, dy)
    ln2 = math.log(2.0)
    np.testing.assert_allclose(gr["dx"].ravel(), e["dx"], atol=1e-14)
    np.testing.assert_allclose(gr["ddt"].ravel(), [4.5, 3 + 1.5 * ln2, -8 + 0.5 * ln2], atol=1e-14)
    np.testing.assert_allclose(gr["dA"], [e["dA"]], atol=1e-14)
    np.testing.assert_allclose(gr["dB"].ravel(), e["dB"], atol=1e-14)
    np.testing.assert_allclose(gr["dC"].ravel(), e["dC"], atol=1e-14)
    np.testing.assert_allclose(gr["dD"], [e["dD"]], atol=1e-14)


@pytest.mark.parametrize("shape", SHAPES)
def test_sequential_matches_dual_form(shape):
    inp, _ = rand_inputs(10, *shape)
    y, _ = seq.ssd_fwd(**inp)
    assert rel(y, dual.ssd_fwd_dual(**inp)) < 1e-13


@pytest.mark.parametrize("shape", SHAPES)
def test_chunked_matches_sequential(shape):
    inp, dy = rand_inputs(11, *shape)
    y, fs = seq.ssd_fwd(**inp)
    g = seq.ssd_bwd(**inp, dy=dy)
    L = shape[1]
    for Q in [q for q in range(1, L + 1) if L % q == 0]:
        o = chunked.ssd_chunked(**inp, chunk=Q, dy=dy)
        assert rel(o["y"], y) < 1e-13, Q
        assert rel(o["final_state"], fs) < 1e-13, Q
        for k, v in g.items():
            assert rel(o[k], v) < 1e-12, (Q, k)


@pytest.mark.parametrize("shape", SHAPES[1:])
def test_finite_differences_all_gradients(shape):
    inp, dy = rand_inputs(12, *shape)
    g = seq.ssd_bwd(**inp, dy=dy)
    f = lambda **kw: seq.ssd_fwd(**kw)[0]
    rng = np.random.default_rng(0)
    for name in ["x", "dt", "A", "B", "C", "D"]:
        arr = inp[name]
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            num = fd.central_diff(f, inp, name, idx, dy, eps=1e-6)
            an = g["d" + name][idx]
            scale = max(1.0, np.abs(g["d" + name]).max())
            assert abs(num - an) / scale < 1e-7, (name, idx, num, an)


def test_length_one_closed_form():
    inp, dy = rand_inputs(13, 2, 1, 3, 4, 5, 1)
    y, fs = seq.ssd_fwd(**inp)
    x, dt, B, C, D = inp["x"], inp["dt"], inp["B"], inp["C"], inp["D"]
    cb = np.einsum("bgn,bgn->bg", C[:, 0], B[:, 0])[:, 0]
    want = dt[:, 0, :, None] * cb[:, None, None] * x[:, 0] + D[None, :, None] * x[:, 0]
    assert rel(y[:, 0], want) < 1e-14
    want_fs = np.einsum("bh,bhp,bn->bhpn", dt[:, 0], x[:, 0], B[:, 0, 0])
    assert rel(fs, want_fs) < 1e-14


def test_zero_decay_is_cumulative_linear_attention():
    inp, dy = rand_inputs(14, 1, 20, 2, 3, 4, 1)
    inp["A"] = np.zeros(2)
    y, fs = seq.ssd_fwd(**inp)
    x, dt, B, C, D = inp["x"][0], inp["dt"][0], inp["B"][0, :, 0], inp["C"][0, :, 0], inp["D"]
    for h in range(2):
        Sc = np.cumsum(dt[:, h, None, None] * B[:, :, None] * x[:, h, None, :], axis=0)  # [t, n, p]
        want = np.einsum("tn,tnp->tp", C, Sc) + D[h] * x[:, h]
        assert rel(y[0, :, h], want) < 1e-13


def test_memoryless_limit():
    inp, dy = rand_inputs(15, 1, 10, 2, 3, 4, 1, dt_scale=1.0)
    inp["dt"] = inp["dt"] + 0.1
    inp["A"] = np.full(2, -1e4)  # exp(dt A) == 0 exactly in float64
    y, _ = seq.ssd_fwd(**inp)
    g = seq.ssd_bwd(**inp, dy=dy)
    x, dt, B, C, D = inp["x"], inp["dt"], inp["B"][:, :, 0], inp["C"][:, :, 0], inp["D"]
    cb = np.einsum("btn,btn->bt", C, B)
    want = dt[..., None] * cb[:, :, None, None] * x + D[None, None, :, None] * x
    assert rel(y, want) < 1e-14
    assert rel(g["dx"], dt[..., None] * cb[:, :, None, None] * dy + D[None, None, :, None] * dy) < 1e-14
    xdy = np.einsum("bthp,bthp->bth", x, dy)
    assert rel(g["dC"][:, :, 0], np.einsum("bth,btn->btn", dt * xdy, B)) < 1e-14
    assert rel(g["dB"][:, :, 0], np.einsum("bth,btn->btn", dt * xdy, C)) < 1e-14
    assert rel(g["ddt"], cb[:, :, None] * xdy) < 1e-14
    assert np.all(g["dA"] == 0.0)


def test_scalar_state_is_first_order_iir_filter():
    # N = P = 1 and a constant step: S_t = a S_{t-1} + u_t, a first-order IIR filter.
    rng = np.random.default_rng(16)
    L = 50
    x = rng.standard_normal((1, L, 1, 1))
    dt = np.full((1, L, 1), 0.3)
    A = np.array([-0.7])
    B = rng.standard_normal((1, L, 1, 1))
    C = rng.standard_normal((1, L, 1, 1))
    D = np.array([0.25])
    y, fs = seq.ssd_fwd(x, dt, A, B, C, D)
    a = math.exp(0.3 * -0.7)
    u = 0.3 * B.ravel() * x.ravel()
    S = scipy.signal.lfilter([1.0], [1.0, -a], u)
    assert rel(y.ravel(), C.ravel() * S + 0.25 * x.ravel()) < 1e-13
    assert abs(fs.ravel()[0] - S[-1]) < 1e-13


def test_zero_B_and_zero_x():
    inp, dy = rand_inputs(17, 2, 8, 4, 3, 5, 2)
    zB = dict(inp, B=np.zeros_like(inp["B"]))
    y, fs = seq.ssd_fwd(**zB)
    g = seq.ssd_bwd(**zB, dy=dy)
    assert rel(y, inp["D"][None, None, :, None] * inp["x"]) < 1e-15
    assert np.all(fs == 0) and np.all(g["dC"] == 0) and np.all(g["ddt"] == 0) and np.all(g["dA"] == 0)
    assert rel(g["dx"], inp["D"][None, None, :, None] * dy) < 1e-15
    zx = dict(inp, x=np.zeros_like(inp["x"]))
    y, fs = seq.ssd_fwd(**zx)
    g = seq.ssd_bwd(**zx, dy=dy)
    assert np.all(y == 0) and np.all(fs == 0)
    for k in ["dB", "dC", "ddt", "dA", "dD"]:
        assert np.all(g[k] == 0), k


@pytest.mark.parametrize("shape", SHAPES[1:])
def test_homogeneity_identities(shape):
    """Exact identities from the layer's scaling symmetries:
    (i)   <x_h, dx_h> = <dy_h, y_h>                     (y is linear in x)
    (ii)  D_h dD_h = <dy_h, D_h x_h>
    (iii) <B_g, dB_g> = <C_g, dC_g> = sum_{h in g} <dy_h, y_h - D_h x_h>
    (iv)  sum dt_h ddt_h - A_h dA_h = <dy_h, y_h - D_h x_h>  (dt -> s dt, A -> A / s)"""
    inp, dy = rand_inputs(18, *shape)
    y, _ = seq.ssd_fwd(**inp)
    g = seq.ssd_bwd(**inp, dy=dy)
    x, dt, A, B, C, D = (inp[k] for k in ["x", "dt", "A", "B", "C", "D"])
    H, G = x.shape[2], B.shape[2]
    ysd = y - D[None, None, :, None] * x
    e_h = np.einsum("bthp,bthp->h", dy, ysd)
    np.testing.assert_allclose(np.einsum("bthp,bthp->h", x, g["dx"]), np.einsum("bthp,bthp->h", dy, y), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(D * g["dD"], np.einsum("bthp,bthp->h", dy, D[None, None, :, None] * x), rtol=1e-12, atol=1e-12)
    e_g = e_h.reshape(G, H // G).sum(1)
    np.testing.assert_allclose(np.einsum("btgn,btgn->g", B, g["dB"]), e_g, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(np.einsum("btgn,btgn->g", C, g["dC"]), e_g, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(np.einsum("bth,bth->h", dt, g["ddt"]) - A * g["dA"], e_h, rtol=1e-11, atol=1e-11)


def test_thread_count_does_not_change_results():
    inp, dy = rand_inputs(19, 3, 40, 4, 4, 6, 2)
    a = seq.ssd_bwd(**inp, dy=dy, nthreads=1)
    b = seq.ssd_bwd(**inp, dy=dy, nthreads=4)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    y1, f1 = seq.ssd_fwd(**inp, nthreads=1)
    y4, f4 = seq.ssd_fwd(**inp, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(f1, f4)


def test_checkpointed_reverse_sweep_crosses_segments():
    # seqlen > 256 exercises the oracle's checkpoint/recompute across several segments.
    inp, dy = rand_inputs(20, 1, 600, 2, 2, 3, 1, dt_scale=0.05)
    g = seq.ssd_bwd(**inp, dy=dy)
    o = chunked.ssd_chunked(**inp, chunk=600, dy=dy)
    for k, v in g.items():
        assert rel(o[k], v) < 1e-11, k
