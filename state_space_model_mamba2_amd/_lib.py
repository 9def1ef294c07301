"""ctypes declarations for libssd.so (include/ssd.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssd.so")

SSD_OK, SSD_ERR_INVALID_ARGUMENT, SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_HIP, SSD_ERR_TOO_LARGE = range(6)
SSD_FWD_STATIC_SCRATCH_BYTES = 96 * 1024 * 1024
SSD_F32, SSD_BF16, SSD_FP8 = 0, 1, 2
SSD_DT_SOFTPLUS = 1

KERNELS = ["cumsum_bmm", "chunk_state", "state_passing", "chunk_scan",
           "chunk_state_bwd", "state_passing_bwd", "chunk_scan_bwd", "dw_heads", "bc_final", "da_dd"]
KERNEL_ID = {n: i for i, n in enumerate(KERNELS)}
N_FWD_KERNELS = KERNELS.index("chunk_state_bwd")  # ids below this are launched by ssd_fwd, the rest by ssd_bwd


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


class Saved(ctypes.Structure):
    _fields_ = [("shape", Shape), ("x", ctypes.c_void_p), ("dt", ctypes.c_void_p), ("B", ctypes.c_void_p),
                ("C", ctypes.c_void_p), ("A", ctypes.c_void_p), ("D", ctypes.c_void_p),
                ("saved_ws", ctypes.c_void_p), ("saved_ws_bytes", ctypes.c_size_t)]


class Regions(ctypes.Structure):
    """Byte offsets of the chunked algorithm's intermediates (ssd_regions)."""
    _fields_ = [("cs", ctypes.c_size_t), ("step", ctypes.c_size_t), ("hin", ctypes.c_size_t),
                ("chunk_state", ctypes.c_size_t), ("dhloc", ctypes.c_size_t), ("gstate", ctypes.c_size_t)]


class ConvShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("channels", ctypes.c_int64),
                ("width", ctypes.c_int32), ("dtype", ctypes.c_int32), ("silu", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class Probe(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("start", ctypes.c_void_p), ("stop", ctypes.c_void_p)]


class LibraryMissing(RuntimeError):
    pass


_lib = None


def load():
    """Load libssd.so from the package directory; raise if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(f"{LIB_PATH} not found: build it with `python -m state_space_model_mamba2_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    PShape, PSaved, PProbe = ctypes.POINTER(Shape), ctypes.POINTER(Saved), ctypes.POINTER(Probe)
    for name in ["ssd_saved_bytes", "ssd_fwd_scratch_bytes", "ssd_bwd_scratch_bytes"]:
        f = getattr(lib, name)
        f.argtypes, f.restype = [PShape], sz
    lib.ssd_check_shape.argtypes, lib.ssd_check_shape.restype = [PShape], st
    lib.ssd_workspace_regions.argtypes = [PShape, ctypes.POINTER(Regions)]
    lib.ssd_workspace_regions.restype = st
    lib.ssd_fwd.argtypes = [PShape, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, PSaved, vp, sz, vp, PProbe]
    lib.ssd_fwd.restype = st
    lib.ssd_fwd_noalloc.argtypes = [PShape, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, PSaved, vp, PProbe]
    lib.ssd_fwd_noalloc.restype = st
    lib.ssd_bwd.argtypes = [PSaved, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, PProbe]
    lib.ssd_bwd.restype = st
    PConv = ctypes.POINTER(ConvShape)
    lib.ssd_conv1d_check_shape.argtypes, lib.ssd_conv1d_check_shape.restype = [PConv], st
    lib.ssd_conv1d_bwd_scratch_bytes.argtypes, lib.ssd_conv1d_bwd_scratch_bytes.restype = [PConv], sz
    lib.ssd_conv1d_fwd.argtypes = [PConv, vp, vp, vp, vp, vp, vp]
    lib.ssd_conv1d_fwd.restype = st
    lib.ssd_conv1d_bwd.argtypes = [PConv, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssd_conv1d_bwd.restype = st
    lib.ssd_status_string.argtypes, lib.ssd_status_string.restype = [st], ctypes.c_char_p
    lib.ssd_kernel_name.argtypes, lib.ssd_kernel_name.restype = [ctypes.c_int32], ctypes.c_char_p
    lib.ssd_version.argtypes, lib.ssd_version.restype = [], ctypes.c_char_p
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().ssd_status_string(code).decode()


def make_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, flags=0) -> Shape:
    return Shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, flags)
