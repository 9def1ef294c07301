"""ctypes wrapper of ssd_oracle.c: the sequential float64 recurrence.

TEST INFRASTRUCTURE (see the package docstring).  Arrays are float64 numpy
arrays in the layouts x/dy [b][L][H][P], dt [b][L][H], B/C [b][L][G][N],
A/D [H]; final_state is [b][H][P][N].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (float64, OpenMP)."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
        tmp = LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                        "-ffp-contract=off", _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(LIB_PATH)
        i64, dp, ci = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.c_int
        lib.oracle_ssd_fwd.argtypes = [i64] * 6 + [dp] * 8 + [ci]
        lib.oracle_ssd_fwd.restype = ci
        lib.oracle_ssd_bwd.argtypes = [i64] * 6 + [dp] * 13 + [ci]
        lib.oracle_ssd_bwd.restype = ci
        lib.oracle_max_threads.restype = ci
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _dims(x, B):
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return b, L, H, P, N, G


def ssd_fwd(x, dt, A, B, C, D, nthreads: int = 0):
    """y [b,L,H,P] and final_state [b,H,P,N] of the sequential recurrence."""
    x, dt, A, B, C, D = map(_f64, (x, dt, A, B, C, D))
    b, L, H, P, N, G = _dims(x, B)
    y = np.empty_like(x)
    fs = np.empty((b, H, P, N), dtype=np.float64)
    rc = _load().oracle_ssd_fwd(b, L, H, P, N, G, _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D),
                                _p(y), _p(fs), nthreads)
    if rc:
        raise RuntimeError(f"oracle_ssd_fwd failed ({rc})")
    return y, fs


def ssd_bwd(x, dt, A, B, C, D, dy, nthreads: int = 0):
    """Gradients (dx, ddt, dA, dB, dC, dD) of <dy, y> w.r.t. the inputs."""
    x, dt, A, B, C, D, dy = map(_f64, (x, dt, A, B, C, D, dy))
    b, L, H, P, N, G = _dims(x, B)
    dx = np.empty_like(x)
    ddt = np.empty_like(dt)
    dA = np.empty_like(A)
    dB = np.empty_like(B)
    dC = np.empty_like(C)
    dD = np.empty_like(D)
    rc = _load().oracle_ssd_bwd(b, L, H, P, N, G, _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D), _p(dy),
                                _p(dx), _p(ddt), _p(dA), _p(dB), _p(dC), _p(dD), nthreads)
    if rc:
        raise RuntimeError(f"oracle_ssd_bwd failed ({rc})")
    return dict(dx=dx, ddt=ddt, dA=dA, dB=dB, dC=dC, dD=dD)
