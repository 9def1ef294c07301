"""The C ABI of libssd on the host: the library loads, exports every function
include/ssd.h declares, and rejects bad arguments before launching anything
(these calls never reach the GPU, so they run without one)."""
import ctypes
import os
import re

import pytest

from state_space_model_mamba2_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = (_lib.SSD_OK, _lib.SSD_ERR_INVALID_ARGUMENT,
                                       _lib.SSD_ERR_UNSUPPORTED, _lib.SSD_ERR_WORKSPACE)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ssd_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"ssd_fwd", "ssd_bwd", "ssd_saved_bytes", "ssd_fwd_scratch_bytes", "ssd_bwd_scratch_bytes",
            "ssd_check_shape", "ssd_status_string", "ssd_kernel_name", "ssd_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def shape(**kw):
    d = dict(batch=2, seqlen=512, nheads=4, headdim=64, dstate=128, ngroups=2, chunk=256, dtype=_lib.SSD_BF16)
    d.update(kw)
    return _lib.make_shape(**d)


def check(lib, s):
    return lib.ssd_check_shape(ctypes.byref(s))


def test_shape_checks(lib):
    assert check(lib, shape()) == OK
    assert check(lib, shape(dtype=_lib.SSD_F32, chunk=64)) == OK
    assert check(lib, shape(chunk=64)) == UNSUPPORTED                        # bf16 chunk 64 switched off
    assert check(lib, shape(dtype=_lib.SSD_F32, chunk=128, dstate=64)) == OK
    assert check(lib, shape(dtype=_lib.SSD_FP8)) == OK and check(lib, shape(dtype=_lib.SSD_FP8, chunk=64)) == UNSUPPORTED
    assert check(lib, shape(seqlen=500)) == OK               # shorter last chunk
    assert check(lib, shape(seqlen=7)) == OK                 # a single, shorter chunk
    assert check(lib, shape(nheads=5)) == INVALID            # nheads % ngroups
    for k in ["batch", "seqlen", "nheads", "headdim", "dstate", "ngroups", "chunk"]:
        assert check(lib, shape(**{k: 0})) == INVALID, k
        assert check(lib, shape(**{k: -1})) == INVALID, k
    assert check(lib, shape(dtype=7)) == INVALID
    assert check(lib, shape(headdim=48)) == UNSUPPORTED
    assert check(lib, shape(dstate=96)) == UNSUPPORTED
    assert check(lib, shape(chunk=32, seqlen=512)) == UNSUPPORTED
    assert check(lib, shape(dtype=_lib.SSD_F32, chunk=256)) == UNSUPPORTED  # fp32 LDS staging limit
    assert check(lib, shape(dtype=_lib.SSD_F32, chunk=128)) == UNSUPPORTED
    s = shape()
    s.flags = 2                                              # unknown flag
    assert check(lib, s) == INVALID
    s.flags = _lib.SSD_DT_SOFTPLUS
    assert check(lib, s) == OK


def test_workspace_sizes(lib):
    s = shape()
    b, L, H, P, N, G, Q = 2, 512, 4, 64, 128, 2, 256
    K = L // Q
    saved = lib.ssd_saved_bytes(ctypes.byref(s))
    assert saved >= 2 * b * H * K * Q * 4 + b * K * H * P * N * 2  # cs, float32 step, Hin
    # chunk states (forward) and dH_loc, G (backward) in the storage dtype (bf16 here)
    assert lib.ssd_fwd_scratch_bytes(ctypes.byref(s)) >= b * K * H * P * N * 2
    assert lib.ssd_bwd_scratch_bytes(ctypes.byref(s)) >= b * K * H * P * N * (2 + 2) + b * K * G * Q * Q * 4
    assert lib.ssd_saved_bytes(ctypes.byref(shape(nheads=5))) == 0
    # a shorter last chunk runs on zero-padded copies: those of x, B, C are
    # kept from the forward to the backward
    ragged = lib.ssd_saved_bytes(ctypes.byref(shape(seqlen=500)))
    assert ragged >= saved + b * Q * (H * P + 2 * G * N) * 2
    for f in (lib.ssd_saved_bytes, lib.ssd_fwd_scratch_bytes, lib.ssd_bwd_scratch_bytes):
        assert f(ctypes.byref(shape(seqlen=7))) > 0
    # with the softplus step the backward adds per-chunk bias-gradient partials
    sp = shape()
    sp.flags = _lib.SSD_DT_SOFTPLUS
    assert lib.ssd_saved_bytes(ctypes.byref(sp)) == saved
    assert lib.ssd_bwd_scratch_bytes(ctypes.byref(sp)) >= lib.ssd_bwd_scratch_bytes(ctypes.byref(s)) + b * K * H * 4
    # sizes grow linearly with batch
    assert lib.ssd_saved_bytes(ctypes.byref(shape(batch=4))) > saved


def test_workspace_regions(lib):
    # each intermediate lies inside the workspace its field names, with room
    # for its array, and no two arrays of one workspace overlap
    for kw in [{}, dict(seqlen=500), dict(dtype=_lib.SSD_F32, chunk=64), dict(dtype=_lib.SSD_FP8, batch=3)]:
        s = shape(**kw)
        r = _lib.Regions()
        assert lib.ssd_workspace_regions(ctypes.byref(s), ctypes.byref(r)) == OK
        b, L, H, P, N, Q = s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.chunk
        K = -(-L // Q)
        esz = 4 if s.dtype == _lib.SSD_F32 else 2
        scal, states = b * H * K * Q * 4, b * K * H * P * N * esz
        spans = {"saved": [(r.cs, scal), (r.step, scal), (r.hin, states)], "fwd": [(r.chunk_state, states)],
                 "bwd": [(r.dhloc, states), (r.gstate, states)]}
        size = {"saved": lib.ssd_saved_bytes(ctypes.byref(s)), "fwd": lib.ssd_fwd_scratch_bytes(ctypes.byref(s)),
                "bwd": lib.ssd_bwd_scratch_bytes(ctypes.byref(s))}
        for ws, sp in spans.items():
            sp = sorted(sp)
            assert all(o % 16 == 0 and o + n <= size[ws] for o, n in sp), (kw, ws, sp)
            assert all(sp[i][0] + sp[i][1] <= sp[i + 1][0] for i in range(len(sp) - 1)), (kw, ws, sp)
    r = _lib.Regions()
    assert lib.ssd_workspace_regions(ctypes.byref(shape(nheads=5)), ctypes.byref(r)) == INVALID
    assert lib.ssd_workspace_regions(ctypes.byref(shape(headdim=48)), ctypes.byref(r)) == UNSUPPORTED
    assert lib.ssd_workspace_regions(ctypes.byref(shape()), None) == INVALID
    assert lib.ssd_workspace_regions(None, ctypes.byref(r)) == INVALID


FAKE = 0x100000  # aligned, never dereferenced: every call below fails validation first


def fwd(lib, s, **over):
    args = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=FAKE, bias=None, s0=None, y=FAKE, fs=FAKE, ws=FAKE,
                ws_bytes=0, scratch=FAKE, scratch_bytes=0)
    args.update(over)
    return lib.ssd_fwd(ctypes.byref(s), args["x"], args["dt"], args["A"], args["B"], args["C"], args["D"],
                       args["bias"], args["s0"], args["y"], args["fs"], args["ws"], args["ws_bytes"], None, args["scratch"],
                       args["scratch_bytes"], None, None)


def test_fwd_rejects_before_launch(lib):
    s = shape()
    need_ws = lib.ssd_saved_bytes(ctypes.byref(s))
    need_scr = lib.ssd_fwd_scratch_bytes(ctypes.byref(s))
    assert fwd(lib, shape(nheads=5)) == INVALID
    assert fwd(lib, shape(headdim=48)) == UNSUPPORTED
    for k in ["x", "dt", "A", "B", "C", "D", "y"]:
        assert fwd(lib, s, **{k: None}, ws_bytes=need_ws, scratch_bytes=need_scr) == INVALID, k
    assert fwd(lib, s, x=FAKE + 8, ws_bytes=need_ws, scratch_bytes=need_scr) == INVALID  # misaligned
    assert fwd(lib, s, s0=FAKE + 4, ws_bytes=need_ws, scratch_bytes=need_scr) == INVALID
    assert fwd(lib, s, bias=FAKE + 4, ws_bytes=need_ws, scratch_bytes=need_scr) == INVALID
    assert fwd(lib, s, ws_bytes=need_ws - 1, scratch_bytes=need_scr) == WORKSPACE
    assert fwd(lib, s, ws=None, ws_bytes=need_ws, scratch_bytes=need_scr) == WORKSPACE
    assert fwd(lib, s, ws_bytes=need_ws, scratch_bytes=need_scr - 1) == WORKSPACE
    assert fwd(lib, s, ws_bytes=need_ws, scratch=None, scratch_bytes=need_scr) == WORKSPACE
    assert lib.ssd_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 0, None, FAKE, 0,
                       None, None) == INVALID


def test_fwd_noalloc_rejects_before_launch(lib):
    # the no-allocation forward checks its arguments like ssd_fwd, and a problem
    # whose forward scratch exceeds the static buffer before it touches the GPU
    def fwd_na(s, ws_bytes, **over):
        a = dict(x=FAKE, y=FAKE, ws=FAKE, s0=None)
        a.update(over)
        return lib.ssd_fwd_noalloc(ctypes.byref(s) if s is not None else None, a["x"], FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None, a["s0"], a["y"], FAKE, a["ws"], ws_bytes, None, None, None)

    s = shape()
    need_ws = lib.ssd_saved_bytes(ctypes.byref(s))
    assert fwd_na(None, 0) == INVALID
    assert fwd_na(shape(nheads=5), need_ws) == INVALID
    assert fwd_na(shape(headdim=48), need_ws) == UNSUPPORTED
    assert fwd_na(s, need_ws, x=None) == INVALID and fwd_na(s, need_ws, y=None) == INVALID
    assert fwd_na(s, need_ws, x=FAKE + 8) == INVALID and fwd_na(s, need_ws, s0=FAKE + 4) == INVALID
    assert fwd_na(s, need_ws - 1) == WORKSPACE and fwd_na(s, need_ws, ws=None) == WORKSPACE
    # the long-context shape (1 x 65536 tokens, 80 heads of 64 x 128, bf16) needs 320 MiB of chunk states
    big = shape(batch=1, seqlen=65536, nheads=80, ngroups=8)
    assert lib.ssd_fwd_scratch_bytes(ctypes.byref(big)) > _lib.SSD_FWD_STATIC_SCRATCH_BYTES
    assert fwd_na(big, lib.ssd_saved_bytes(ctypes.byref(big))) == _lib.SSD_ERR_TOO_LARGE
    # the 2.7B shape fits (80 MiB)
    fits = shape(batch=4, seqlen=4096, nheads=80, ngroups=1)
    assert lib.ssd_fwd_scratch_bytes(ctypes.byref(fits)) <= _lib.SSD_FWD_STATIC_SCRATCH_BYTES
    assert "static buffer" in _lib.status_string(_lib.SSD_ERR_TOO_LARGE)


def test_bwd_rejects_before_launch(lib):
    s = shape()
    sv = _lib.Saved(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, lib.ssd_saved_bytes(ctypes.byref(s)))
    need = lib.ssd_bwd_scratch_bytes(ctypes.byref(s))

    def bwd(saved, dy=FAKE, scratch=FAKE, nbytes=need, dx=FAKE, dfs=None, ds0=None, dbias=None):
        return lib.ssd_bwd(ctypes.byref(saved) if saved is not None else None, dy, dfs, dx, FAKE, FAKE, FAKE, FAKE,
                           FAKE, dbias, ds0, scratch, nbytes, None, None)

    assert bwd(None) == INVALID
    assert bwd(sv, dy=None) == INVALID
    assert bwd(sv, dx=None) == INVALID
    assert bwd(sv, dfs=FAKE + 4) == INVALID  # misaligned optional state pointers
    assert bwd(sv, ds0=FAKE + 8) == INVALID
    assert bwd(sv, dbias=FAKE + 8) == INVALID
    assert bwd(sv, nbytes=need - 1) == WORKSPACE
    assert bwd(sv, scratch=None) == WORKSPACE
    small = _lib.Saved(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16)
    assert bwd(small) == WORKSPACE
    bad = _lib.Saved(shape(nheads=5), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30)
    assert bwd(bad) == INVALID
    fp8 = _lib.Saved(shape(dtype=_lib.SSD_FP8), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30)
    need8 = lib.ssd_bwd_scratch_bytes(ctypes.byref(fp8.shape))
    assert need8 > 0 and bwd(fp8, nbytes=need8 - 1) == WORKSPACE   # FP8 operands: checked like bf16
    assert bwd(fp8, dy=None, nbytes=need8) == INVALID


def test_strings(lib):
    assert lib.ssd_version().decode().count(".") == 2
    for code in range(6):
        assert lib.ssd_status_string(code)
    for i, n in enumerate(_lib.KERNELS):
        assert lib.ssd_kernel_name(i).decode() == n
    assert lib.ssd_kernel_name(len(_lib.KERNELS)) is None
    assert lib.ssd_kernel_name(-1) is None


def conv_shape(**kw):
    d = dict(batch=2, seqlen=100, channels=64, width=4, dtype=_lib.SSD_BF16, silu=1, reserved=0)
    d.update(kw)
    return _lib.ConvShape(**d)


def test_conv_shape_checks_and_rejections(lib):
    chk = lambda s: lib.ssd_conv1d_check_shape(ctypes.byref(s))
    assert chk(conv_shape()) == OK
    assert chk(conv_shape(dtype=_lib.SSD_F32, width=2, silu=0)) == OK
    assert chk(conv_shape(width=5)) == UNSUPPORTED and chk(conv_shape(width=1)) == UNSUPPORTED
    assert chk(conv_shape(channels=66)) == UNSUPPORTED
    for k in ["batch", "seqlen", "channels"]:
        assert chk(conv_shape(**{k: 0})) == INVALID, k
    assert chk(conv_shape(silu=2)) == INVALID and chk(conv_shape(reserved=1)) == INVALID
    assert chk(conv_shape(dtype=9)) == INVALID
    s = conv_shape()
    need = lib.ssd_conv1d_bwd_scratch_bytes(ctypes.byref(s))
    assert need >= 2 * 64 * 5 * 4
    assert lib.ssd_conv1d_fwd(ctypes.byref(s), None, FAKE, None, None, FAKE, None) == INVALID
    assert lib.ssd_conv1d_fwd(ctypes.byref(s), FAKE + 4, FAKE, None, None, FAKE, None) == INVALID
    bwd = lambda scratch, nbytes, dx=FAKE: lib.ssd_conv1d_bwd(ctypes.byref(s), FAKE, FAKE, None, None, FAKE, dx, FAKE,
                                                               None, None, scratch, nbytes, None)
    assert bwd(FAKE, need, dx=None) == INVALID
    assert bwd(FAKE, need - 1) == WORKSPACE and bwd(None, need) == WORKSPACE
