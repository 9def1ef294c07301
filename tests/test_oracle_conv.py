"""Pins for the causal depthwise conv1d oracle (CPU only).

* torch.nn.functional.conv1d (depthwise, groups = channels, left-padded) in
  float64 for the pre-activation, and torch's autograd through it and SiLU
  for every gradient;
* scipy.signal.lfilter as a causal FIR filter, channel by channel;
* central finite differences of <dy, y> for x, w, bias and x_prev;
* special filters: a unit tap at the last position (y = act(x + bias)) and
  at the first (a delay by W - 1 rows);
* splitting the sequence with the halo x_prev equals one run, forward and
  backward.
"""
import numpy as np
import pytest
import scipy.signal

from oracle import conv, fd

torch = pytest.importorskip("torch")


def draw(seed, b, L, C, W):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((b, L, C)), rng.standard_normal((C, W)) / W, rng.standard_normal(C) * 0.1,
            rng.standard_normal((b, W - 1, C)), rng.standard_normal((b, L, C)))


@pytest.mark.parametrize("W", [2, 3, 4])
@pytest.mark.parametrize("silu", [False, True])
def test_matches_torch_conv1d_and_autograd(W, silu):
    b, L, C = 2, 19, 5
    x, w, bias, prev, dy = draw(60 + W, b, L, C, W)
    y = conv.conv1d_fwd(x, w, bias, prev, silu=silu)
    g = conv.conv1d_bwd(x, w, dy, bias, prev, silu=silu)
    tx = torch.tensor(x, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    tb = torch.tensor(bias, requires_grad=True)
    tp = torch.tensor(prev, requires_grad=True)
    inp = torch.cat([tp, tx], dim=1).transpose(1, 2)                    # [b, C, L + W - 1]
    z = torch.nn.functional.conv1d(inp, tw[:, None, :], tb, groups=C)  # valid conv: L outputs
    ty = torch.nn.functional.silu(z) if silu else z
    ty = ty.transpose(1, 2)
    assert np.max(np.abs(ty.detach().numpy() - y)) < 1e-13
    (ty * torch.tensor(dy)).sum().backward()
    for name, t in (("dx", tx), ("dw", tw), ("dbias", tb), ("dx_prev", tp)):
        assert np.max(np.abs(t.grad.numpy() - g[name])) < 1e-12, name


def test_is_a_causal_fir_filter():
    b, L, C, W = 1, 40, 3, 4
    x, w, bias, _, _ = draw(70, b, L, C, W)
    y = conv.conv1d_fwd(x, w, bias, silu=False)
    for c in range(C):
        want = scipy.signal.lfilter(w[c][::-1], [1.0], x[0, :, c]) + bias[c]
        assert np.max(np.abs(y[0, :, c] - want)) < 1e-13


@pytest.mark.parametrize("silu", [False, True])
def test_finite_differences(silu):
    b, L, C, W = 2, 9, 3, 4
    x, w, bias, prev, dy = draw(71, b, L, C, W)
    g = conv.conv1d_bwd(x, w, dy, bias, prev, silu=silu)
    f = lambda x, w, bias, x_prev: conv.conv1d_fwd(x, w, bias, x_prev, silu=silu)
    vals = dict(x=x, w=w, bias=bias, x_prev=prev)
    grads = dict(x="dx", w="dw", bias="dbias", x_prev="dx_prev")
    rng = np.random.default_rng(72)
    for name, gname in grads.items():
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in vals[name].shape)
            num = fd.central_diff(f, vals, name, idx, dy, eps=1e-6)
            assert abs(num - g[gname][idx]) < 1e-7 * max(1.0, np.abs(g[gname]).max()), (name, idx)


def test_special_filters():
    b, L, C, W = 2, 12, 4, 4
    x, _, bias, _, _ = draw(73, b, L, C, W)
    unit_last = np.zeros((C, W))
    unit_last[:, -1] = 1.0
    z = x + bias
    assert np.max(np.abs(conv.conv1d_fwd(x, unit_last, bias) - z / (1 + np.exp(-z)))) < 1e-14
    unit_first = np.zeros((C, W))
    unit_first[:, 0] = 1.0
    y = conv.conv1d_fwd(x, unit_first, None, silu=False)
    assert np.all(y[:, :W - 1] == 0) and np.array_equal(y[:, W - 1:], x[:, :L - (W - 1)])


def test_split_with_halo_equals_one_run():
    b, L, C, W = 2, 20, 3, 4
    x, w, bias, prev, dy = draw(74, b, L, C, W)
    cut = 7
    y = conv.conv1d_fwd(x, w, bias, prev)
    g = conv.conv1d_bwd(x, w, dy, bias, prev)
    y1 = conv.conv1d_fwd(x[:, :cut], w, bias, prev)
    y2 = conv.conv1d_fwd(x[:, cut:], w, bias, x[:, cut - (W - 1):cut])
    assert np.max(np.abs(np.concatenate([y1, y2], 1) - y)) < 1e-14
    g1 = conv.conv1d_bwd(x[:, :cut], w, dy[:, :cut], bias, prev)
    g2 = conv.conv1d_bwd(x[:, cut:], w, dy[:, cut:], bias, x[:, cut - (W - 1):cut])
    dx = np.concatenate([g1["dx"], g2["dx"]], 1)
    dx[:, cut - (W - 1):cut] += g2["dx_prev"]            # the halo's gradient flows back to its rows
    assert np.max(np.abs(dx - g["dx"])) < 1e-13
    assert np.max(np.abs(g1["dw"] + g2["dw"] - g["dw"])) < 1e-12
    assert np.max(np.abs(g1["dbias"] + g2["dbias"] - g["dbias"])) < 1e-12
    assert np.max(np.abs(g1["dx_prev"] - g["dx_prev"])) < 1e-14
