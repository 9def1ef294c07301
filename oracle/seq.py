"""ctypes wrapper of ssd_oracle.c: the sequential float64 recurrence.

TEST INFRASTRUCTURE (see the package docstring).  Arrays are float64 numpy
arrays in the layouts x/dy [b][L][H][P], dt [b][L][H], B/C [b][L][G][N],
A/D [H]; final_state, initial_state, dinitial_state and dfinal_state are
[b][H][P][N] (element [p][n] is the state's entry [n][p]).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
# SSD_ORACLE_LIB names another build of the same source (the sanitizer test
# loads one built with AddressSanitizer); it is used as is, never rebuilt here.
LIB_PATH = os.environ.get("SSD_ORACLE_LIB") or os.path.join(_HERE, "libssd_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (float64, OpenMP)."""
    if os.environ.get("SSD_ORACLE_LIB"):
        return LIB_PATH
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
        lib.oracle_ssd_fwd.argtypes = [i64] * 6 + [dp] * 9 + [ci]
        lib.oracle_ssd_fwd.restype = ci
        lib.oracle_ssd_bwd.argtypes = [i64] * 6 + [dp] * 16 + [ci]
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


def _state(a, b, H, P, N):
    if a is None:
        return None
    a = _f64(a)
    if a.shape != (b, H, P, N):
        raise ValueError(f"state must have shape {(b, H, P, N)}, got {a.shape}")
    return a


def _pn(a):
    return _p(a) if a is not None else None


def ssd_fwd(x, dt, A, B, C, D, initial_state=None, nthreads: int = 0):
    """y [b,L,H,P] and final_state [b,H,P,N] of the sequential recurrence
    started from initial_state (zero if None)."""
    x, dt, A, B, C, D = map(_f64, (x, dt, A, B, C, D))
    b, L, H, P, N, G = _dims(x, B)
    s0 = _state(initial_state, b, H, P, N)
    y = np.empty_like(x)
    fs = np.empty((b, H, P, N), dtype=np.float64)
    rc = _load().oracle_ssd_fwd(b, L, H, P, N, G, _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D),
                                _pn(s0), _p(y), _p(fs), nthreads)
    if rc:
        raise RuntimeError(f"oracle_ssd_fwd failed ({rc})")
    return y, fs


def ssd_bwd(x, dt, A, B, C, D, dy, initial_state=None, dfinal_state=None, nthreads: int = 0):
    """Gradients (dx, ddt, dA, dB, dC, dD, dinitial_state) of
    <dy, y> + <dfinal_state, final_state> w.r.t. the inputs, for the
    recurrence started from initial_state (None means zero for both)."""
    x, dt, A, B, C, D, dy = map(_f64, (x, dt, A, B, C, D, dy))
    b, L, H, P, N, G = _dims(x, B)
    s0 = _state(initial_state, b, H, P, N)
    dfs = _state(dfinal_state, b, H, P, N)
    ds0 = np.empty((b, H, P, N), dtype=np.float64)
    dx = np.empty_like(x)
    ddt = np.empty_like(dt)
    dA = np.empty_like(A)
    dB = np.empty_like(B)
    dC = np.empty_like(C)
    dD = np.empty_like(D)
    rc = _load().oracle_ssd_bwd(b, L, H, P, N, G, _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D), _p(dy),
                                _pn(s0), _pn(dfs), _p(dx), _p(ddt), _p(dA), _p(dB), _p(dC), _p(dD),
                                _p(ds0), nthreads)
    if rc:
        raise RuntimeError(f"oracle_ssd_bwd failed ({rc})")
    return dict(dx=dx, ddt=ddt, dA=dA, dB=dB, dC=dC, dD=dD, dinitial_state=ds0)
