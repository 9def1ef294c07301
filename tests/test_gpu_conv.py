"""libssd's causal depthwise conv1d on the GPU against the float64 oracle.

Tolerance: per tensor max|gpu - oracle| / max|oracle| <= 1e-4 (fp32 storage)
or 2e-2 (bf16 storage, fp32 arithmetic), as for the scan.  Channels are
independent, so at full size the oracle runs on a sample of channels (every
token, every batch row) and the comparison is exact for those.
"""
import numpy as np
import pytest

from state_space_model_mamba2_amd import inputs
from tests.util import max_rel, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_gpu(ci, silu, with_bias, with_prev):
    from state_space_model_mamba2_amd import ssd

    x, w, dy = _dev(ci.x), _dev(ci.w), _dev(ci.dy)
    bias = _dev(ci.bias) if with_bias else None
    prev = _dev(ci.x_prev) if with_prev else None
    y = ssd.conv1d_fwd(x, w, bias, prev, silu)
    g = ssd.conv1d_bwd(x, w, dy, bias, prev, silu, want_dx_prev=True)
    torch.cuda.synchronize()
    return dict(y=to_np(y), **{k: to_np(v) for k, v in g.items()})


def run_oracle(ci, silu, with_bias, with_prev, ch=slice(None)):
    from oracle import conv

    x, dy = ci.as_f64("x")[:, :, ch], ci.as_f64("dy")[:, :, ch]
    w = ci.as_f64("w")[ch]
    bias = ci.as_f64("bias")[ch] if with_bias else None
    prev = ci.as_f64("x_prev")[:, :, ch] if with_prev else None
    y = conv.conv1d_fwd(x, w, bias, prev, silu)
    g = conv.conv1d_bwd(x, w, dy, bias, prev, silu)
    if not with_bias:
        g.pop("dbias")
    return dict(y=y, **g)


CASES = [  # (batch, seqlen, channels, width, dtype, silu, bias, prev)
    (1, 1, 4, 4, "f32", True, True, True),
    (2, 5, 36, 4, "f32", True, True, False),
    (2, 37, 260, 4, "f32", False, False, True),
    (3, 300, 36, 3, "f32", True, True, True),
    (2, 129, 64, 2, "f32", True, False, False),
    (2, 300, 260, 4, "bf16", True, True, True),
    (1, 17, 36, 2, "bf16", False, True, True),
    (2, 1000, 520, 3, "bf16", True, True, False),
    (4, 257, 1028, 4, "bf16", True, False, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(v) for v in c))
def test_conv_parity(case):
    b, L, C, W, dtype, silu, with_bias, with_prev = case
    print(f"[conv] {case}", flush=True)
    ci = inputs.generate_conv(b, L, C, W, dtype, seed=20)
    got = run_gpu(ci, silu, with_bias, with_prev)
    ref = run_oracle(ci, silu, with_bias, with_prev)
    errs = {k: max_rel(got[k], ref[k]) for k in ref}
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[dtype]}
    assert not bad, (case, bad)


@pytest.mark.parametrize("name", ["mamba2_2p7b", "long_context"])
def test_conv_full_size_sampled_channels(name):
    cw = inputs.CONV_WORKLOADS[name]
    print(f"[conv full] {name}: {cw}", flush=True)
    ci = inputs.generate_conv(cw["batch"], cw["seqlen"], cw["channels"], cw["width"], cw["dtype"], seed=21)
    got = run_gpu(ci, True, True, True)
    C = cw["channels"]
    ch = np.r_[0:32, C // 2:C // 2 + 32, C - 32:C]
    ref = run_oracle(ci, True, True, True, ch)
    sel = dict(y=got["y"][:, :, ch], dx=got["dx"][:, :, ch], dw=got["dw"][ch], dbias=got["dbias"][ch],
               dx_prev=got["dx_prev"][:, :, ch])
    errs = {k: max_rel(sel[k], ref[k]) for k in ref}
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[cw["dtype"]]}
    assert not bad, (name, bad)


def test_conv_split_with_halo():
    """A sequence cut in two: the second piece takes the first's last W-1
    rows as its halo.  Outputs are bitwise those of one call; the halo's
    gradient added to those rows gives dx, and the pieces' dw / dbias add up."""
    from state_space_model_mamba2_amd import ssd

    b, L, C, W = 2, 4096, 5376, 4
    ci = inputs.generate_conv(b, L, C, W, "bf16", seed=22)
    x, w, bias, prev, dy = _dev(ci.x), _dev(ci.w), _dev(ci.bias), _dev(ci.x_prev), _dev(ci.dy)
    y = ssd.conv1d_fwd(x, w, bias, prev)
    g = ssd.conv1d_bwd(x, w, dy, bias, prev, want_dx_prev=True)
    cut = 1501
    x1, x2 = x[:, :cut].contiguous(), x[:, cut:].contiguous()
    halo = x[:, cut - (W - 1):cut].contiguous()
    y1 = ssd.conv1d_fwd(x1, w, bias, prev)
    y2 = ssd.conv1d_fwd(x2, w, bias, halo)
    g1 = ssd.conv1d_bwd(x1, w, dy[:, :cut].contiguous(), bias, prev, want_dx_prev=True)
    g2 = ssd.conv1d_bwd(x2, w, dy[:, cut:].contiguous(), bias, halo, want_dx_prev=True)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([y1, y2], 1), y)
    dx = torch.cat([g1["dx"], g2["dx"]], 1).float()
    dx[:, cut - (W - 1):cut] += g2["dx_prev"].float()
    errs = dict(dx=max_rel(to_np(dx), to_np(g["dx"])), dw=max_rel(to_np(g1["dw"] + g2["dw"]), to_np(g["dw"])),
                dbias=max_rel(to_np(g1["dbias"] + g2["dbias"]), to_np(g["dbias"])),
                dx_prev=max_rel(to_np(g1["dx_prev"]), to_np(g["dx_prev"])))
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert errs["dx_prev"] == 0.0
    assert errs["dx"] <= 1e-2 and errs["dw"] <= 1e-5 and errs["dbias"] <= 1e-5
