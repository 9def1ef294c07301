"""Pins for the oracle's initial state, final-state cotangent and ragged chunking (CPU only).

With an initial state S0 the layer computes y and final_state from the
recurrence started at S_{-1} = S0, and the backward returns the gradients of
<dy, y> + <dS_fin, final_state> together with dS0.  These are pinned by:
  * central finite differences of that scalar for every input, S0 included,
  * a closed form for x = 0: the state is S0 decayed by the running product of
    the per-step decays, so y, final_state, dS0, dC, ddt and dA follow from
    cumulative sums of dt alone,
  * splitting the sequence: two runs chained through the state (forward) and
    through dS0 -> dS_fin (backward) equal one run over the whole sequence,
    which reduces the new arguments to the zero-state path pinned elsewhere,
  * the homogeneity identity of a map that is linear in (x, S0) jointly,
  * the chunked evaluation at every chunk length, including lengths that leave
    a shorter last chunk.
"""
import math

import numpy as np
import pytest

from oracle import chunked, fd, seq
from tests.test_oracle import rand_inputs, rel

SHAPES = [  # b, L, H, P, N, G
    (1, 1, 1, 1, 1, 1),
    (2, 12, 4, 3, 5, 2),
    (1, 17, 3, 2, 4, 1),
]


def states(seed, b, H, P, N):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((b, H, P, N)), rng.standard_normal((b, H, P, N))


@pytest.mark.parametrize("shape", SHAPES)
def test_finite_differences_with_states(shape):
    b, L, H, P, N, G = shape
    inp, dy = rand_inputs(30, *shape)
    s0, dfs = states(31, b, H, P, N)
    inp["initial_state"] = s0
    g = seq.ssd_bwd(**inp, dy=dy, dfinal_state=dfs)

    def f(**kw):  # y and final_state flattened, paired with (dy, dS_fin)
        y, fs = seq.ssd_fwd(**kw)
        return np.concatenate([y.ravel(), fs.ravel()])

    cot = np.concatenate([dy.ravel(), dfs.ravel()])
    rng = np.random.default_rng(1)
    grads = dict(x="dx", dt="ddt", A="dA", B="dB", C="dC", D="dD", initial_state="dinitial_state")
    for name, gname in grads.items():
        arr = inp[name]
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            num = fd.central_diff(f, inp, name, idx, cot, eps=1e-6)
            an = g[gname][idx]
            scale = max(1.0, np.abs(g[gname]).max())
            assert abs(num - an) / scale < 1e-7, (name, idx, num, an)


def test_zero_input_closed_form():
    b, L, H, P, N, G = 2, 15, 4, 3, 5, 2
    inp, dy = rand_inputs(32, b, L, H, P, N, G)
    inp["x"] = np.zeros_like(inp["x"])
    s0, dfs = states(33, b, H, P, N)
    y, fs = seq.ssd_fwd(**inp, initial_state=s0)
    g = seq.ssd_bwd(**inp, dy=dy, initial_state=s0, dfinal_state=dfs)
    dt, A, C = inp["dt"], inp["A"], inp["C"]
    hg = np.arange(H) // (H // G)
    Ch = C[:, :, hg, :]                                    # [b, L, H, N]
    c = np.cumsum(dt, axis=1)                              # [b, L, H]
    dec = np.exp(A * c)                                    # running product of the decays
    S0C = np.einsum("bhpn,blhn->blhp", s0, Ch)
    assert rel(y, dec[..., None] * S0C) < 1e-14
    assert rel(fs, dec[:, -1, :, None, None] * s0) < 1e-14
    want_ds0 = np.einsum("blh,blhp,blhn->bhpn", dec, dy, Ch) + dec[:, -1, :, None, None] * dfs
    assert rel(g["dinitial_state"], want_ds0) < 1e-13
    # loss = sum_t dec_t m_t + dec_{L-1} m_fin with m_t = <dy_t, S0 C_t>, m_fin = <dS_fin, S0>
    m = np.einsum("blhp,blhp->blh", dy, S0C)
    mfin = np.einsum("bhpn,bhpn->bh", dfs, s0)
    contrib = dec * m
    contrib[:, -1] += dec[:, -1] * mfin
    suffix = np.flip(np.cumsum(np.flip(contrib, 1), 1), 1)
    assert rel(g["ddt"], A * suffix) < 1e-13
    assert rel(g["dA"], np.einsum("blh,blh->h", c, contrib)) < 1e-13
    dCh = dec[..., None] * np.einsum("blhp,bhpn->blhn", dy, s0)
    assert rel(g["dC"], dCh.reshape(b, L, G, H // G, N).sum(3)) < 1e-13
    assert np.all(g["dB"] == 0) and np.all(g["dD"] == 0)


@pytest.mark.parametrize("with_s0", [False, True])
@pytest.mark.parametrize("split", [1, 5, 11])
def test_split_sequence_chains_through_the_state(with_s0, split):
    b, L, H, P, N, G = 2, 12, 4, 3, 5, 2
    inp, dy = rand_inputs(34, b, L, H, P, N, G)
    s0, dfs = states(35, b, H, P, N)
    s0 = s0 if with_s0 else None
    dfs = dfs if with_s0 else None
    y, fs = seq.ssd_fwd(**inp, initial_state=s0)
    g = seq.ssd_bwd(**inp, dy=dy, initial_state=s0, dfinal_state=dfs)
    one = {k: v[:, :split] if k not in ("A", "D") else v for k, v in inp.items()}
    two = {k: v[:, split:] if k not in ("A", "D") else v for k, v in inp.items()}
    y1, f1 = seq.ssd_fwd(**one, initial_state=s0)
    y2, f2 = seq.ssd_fwd(**two, initial_state=f1)
    assert rel(np.concatenate([y1, y2], 1), y) < 1e-14
    assert rel(f2, fs) < 1e-14
    g2 = seq.ssd_bwd(**two, dy=dy[:, split:], initial_state=f1, dfinal_state=dfs)
    g1 = seq.ssd_bwd(**one, dy=dy[:, :split], initial_state=s0, dfinal_state=g2["dinitial_state"])
    for k in ("dx", "ddt", "dB", "dC"):
        assert rel(np.concatenate([g1[k], g2[k]], 1), g[k]) < 1e-13, k
    for k in ("dA", "dD"):
        assert rel(g1[k] + g2[k], g[k]) < 1e-13, k
    assert rel(g1["dinitial_state"], g["dinitial_state"]) < 1e-13


def test_linear_in_input_and_initial_state():
    """y and final_state are linear in (x, S0) jointly, so per head
    <x, dx> + <S0, dS0> = <dy, y> + <dS_fin, final_state>."""
    b, L, H, P, N, G = 2, 12, 4, 3, 5, 2
    inp, dy = rand_inputs(36, b, L, H, P, N, G)
    s0, dfs = states(37, b, H, P, N)
    y, fs = seq.ssd_fwd(**inp, initial_state=s0)
    g = seq.ssd_bwd(**inp, dy=dy, initial_state=s0, dfinal_state=dfs)
    lhs = np.einsum("blhp,blhp->h", inp["x"], g["dx"]) + np.einsum("bhpn,bhpn->h", s0, g["dinitial_state"])
    rhs = np.einsum("blhp,blhp->h", dy, y) + np.einsum("bhpn,bhpn->h", dfs, fs)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_no_state_arguments_mean_zero():
    b, L, H, P, N, G = 1, 9, 2, 3, 4, 1
    inp, dy = rand_inputs(38, b, L, H, P, N, G)
    z = np.zeros((b, H, P, N))
    y0, f0 = seq.ssd_fwd(**inp)
    y1, f1 = seq.ssd_fwd(**inp, initial_state=z)
    assert np.array_equal(y0, y1) and np.array_equal(f0, f1)
    g0 = seq.ssd_bwd(**inp, dy=dy)
    g1 = seq.ssd_bwd(**inp, dy=dy, initial_state=z, dfinal_state=z)
    for k in g0:
        assert np.array_equal(g0[k], g1[k]), k


@pytest.mark.parametrize("shape", SHAPES[1:])
def test_chunked_any_chunk_length_matches_sequential(shape):
    b, L, H, P, N, G = shape
    inp, dy = rand_inputs(39, *shape)
    s0, dfs = states(40, b, H, P, N)
    y, fs = seq.ssd_fwd(**inp, initial_state=s0)
    g = seq.ssd_bwd(**inp, dy=dy, initial_state=s0, dfinal_state=dfs)
    for Q in range(1, L + 2):
        o = chunked.ssd_chunked(**inp, chunk=Q, dy=dy, initial_state=s0, dfinal_state=dfs)
        assert rel(o["y"], y) < 1e-13, Q
        assert rel(o["final_state"], fs) < 1e-13, Q
        for k, v in g.items():
            assert rel(o[k], v) < 1e-12, (Q, k)


def test_decay_of_initial_state_matches_exp_of_cumsum():
    # N = P = 1, x = 0: the state is S0 times exp(A * cumsum(dt)), a direct product.
    dt = np.array([[[0.3], [0.1], [0.7], [0.2]]])
    A = np.array([-0.9])
    x = np.zeros((1, 4, 1, 1))
    B = np.ones((1, 4, 1, 1))
    C = np.ones((1, 4, 1, 1))
    D = np.zeros(1)
    s0 = np.full((1, 1, 1, 1), 2.5)
    y, fs = seq.ssd_fwd(x, dt, A, B, C, D, initial_state=s0)
    want = 2.5 * np.exp(-0.9 * np.array([0.3, 0.4, 1.1, 1.3]))
    assert rel(y.ravel(), want) < 1e-15
    assert abs(fs.ravel()[0] - 2.5 * math.exp(-0.9 * 1.3)) < 1e-15
