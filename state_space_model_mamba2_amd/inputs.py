"""Seeded synthetic inputs for the Mamba-2 SSD scan.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the scan's arithmetic, so both the HIP path (through the
binding) and the float64 oracle consume exactly the same values.

Recipe (one draw per tensor, in this order, from numpy's PCG64 generator
``default_rng(seed)``):

    x      ~ N(0, 1)                            [batch, seqlen, nheads, headdim]
    dt_raw ~ N(0, dt_sigma^2), dt_sigma^2 = 0.5 [batch, seqlen, nheads]
    u_bias ~ U[ln lo, ln hi]                    [nheads]   dt_bias = ln(expm1(exp(u_bias)))
    u_A    ~ U[ln 1, ln 16]                     [nheads]   A = -exp(u_A)
    B      ~ N(0, 1)                            [batch, seqlen, ngroups, dstate]
    C      ~ N(0, 1)                            [batch, seqlen, ngroups, dstate]
    D      ~ N(0, 1)                            [nheads]
    dy     ~ N(0, 1)                            [batch, seqlen, nheads, headdim]

    dt = softplus(dt_raw + dt_bias)             (the post-softplus step size)

For runs that take the raw step and apply the softplus themselves, the same
draws also give dt_raw = N(0, dt_sigma^2) rounded like dt (storage dtype) and
dt_bias (float32, [nheads]).

States for the runs that start from a given state or carry a final-state
cotangent come from their own generator, ``default_rng([seed, 1])``, so the
draws above do not move:

    initial_state ~ N(0, 1)                     [batch, nheads, headdim, dstate]
    dfinal_state  ~ N(0, 1)                     [batch, nheads, headdim, dstate]

both float32 in every mode.

The dt parameterisation (softplus of a per-head bias drawn log-uniformly so
that softplus(bias) lies in [lo, hi]) and A = -exp(U[ln 1, ln 16]) follow the
usual Mamba-2 initialisation; they only shape the synthetic workload.

Normal tensors are drawn in float32 (numpy's float32 ziggurat) for speed at
the long-context size; the small per-head tensors are drawn in float64.  Every
tensor is rounded to float32 (round-to-nearest-even); in bf16 mode x, dt, B,
C and dy are then rounded again to bfloat16 (RNE).  A and D always stay float32.
In fp8 mode x, B and C are rounded from float32 to OCP FP8 E4M3 codes (nearest,
ties to even, saturating at +-448) and dt, dy to bfloat16.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# The five workloads: Mamba-2 SSD shapes of the 370M and 2.7B models, a
# Zamba2-7B-like hybrid block, a long-context case and a tiny fp32 case.
WORKLOADS = {
    "tiny_fp32": dict(batch=1, seqlen=256, nheads=2, headdim=16, dstate=16,
                      ngroups=1, chunk=64, dtype="f32", dt_bias_range=(1e-3, 1e-1)),
    "mamba2_370m": dict(batch=8, seqlen=2048, nheads=32, headdim=64, dstate=128,
                        ngroups=1, chunk=256, dtype="bf16", dt_bias_range=(1e-3, 1e-1)),
    "mamba2_2p7b": dict(batch=4, seqlen=4096, nheads=80, headdim=64, dstate=128,
                        ngroups=1, chunk=256, dtype="bf16", dt_bias_range=(1e-3, 1e-1)),
    "zamba2_7b": dict(batch=2, seqlen=4096, nheads=112, headdim=64, dstate=64,
                      ngroups=2, chunk=256, dtype="bf16", dt_bias_range=(1e-3, 1e-1)),
    "long_context": dict(batch=1, seqlen=65536, nheads=80, headdim=64, dstate=128,
                         ngroups=8, chunk=256, dtype="bf16", dt_bias_range=(1e-4, 1e-2)),
}

WORKLOAD_ORDER = ["tiny_fp32", "mamba2_370m", "mamba2_2p7b", "zamba2_7b", "long_context"]


@dataclasses.dataclass(frozen=True)
class Shape:
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str = "bf16"  # "f32" or "bf16": storage dtype of x, dt, B, C, dy
    dt_bias_range: tuple = (1e-3, 1e-1)

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


def workload(name: str, **overrides) -> Shape:
    kw = dict(WORKLOADS[name])
    kw.update(overrides)
    return Shape(**kw)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _e4m3_table() -> np.ndarray:
    """Value of every OCP FP8 E4M3 code (1 sign, 4 exponent bits with bias 7,
    3 mantissa bits; exponent field 0 is subnormal, S.1111.111 is NaN)."""
    c = np.arange(256)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    v = s * v
    v[(c & 0x7F) == 0x7F] = np.nan
    return v


E4M3_VALUES = _e4m3_table()


def e4m3_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact value of each E4M3 code."""
    return E4M3_VALUES[np.asarray(b, dtype=np.uint8)].astype(np.float32)


def f32_to_e4m3_bits(a: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3 value, ties to the even code, saturating at
    +-448 (the largest finite value); returns uint8 codes."""
    a = np.asarray(a, dtype=np.float64)
    pos = E4M3_VALUES[:0x7F]                      # codes 0x00 .. 0x7E, increasing
    mag = np.minimum(np.abs(a), pos[-1])
    hi = np.clip(np.searchsorted(pos, mag, side="left"), 0, len(pos) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = mag - pos[lo], pos[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(mag == pos[hi], hi, code).astype(np.uint8)
    return np.where(np.signbit(a), code | 0x80, code).astype(np.uint8)  # the sign survives rounding to zero


@dataclasses.dataclass
class Inputs:
    """One seeded draw.  Tensors are numpy arrays in their storage form:
    float32 arrays in f32 mode; uint16 bfloat16 bit patterns in bf16 mode
    (x, dt, B, C, dy); in fp8 mode uint8 E4M3 codes for x, B, C and bfloat16
    bits for dt, dy.  A and D are always float32."""
    shape: Shape
    x: np.ndarray
    dt: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    D: np.ndarray
    dy: np.ndarray
    dt_raw: np.ndarray = None   # pre-softplus step (storage dtype), same draws as dt
    dt_bias: np.ndarray = None  # float32 [nheads]

    def as_f64(self, name: str) -> np.ndarray:
        """Exact float64 view of a tensor's stored values (for the oracle)."""
        a = getattr(self, name)
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a).astype(np.float64)
        if a.dtype == np.uint8:
            return E4M3_VALUES[a]
        return a.astype(np.float64)


def _softplus(v: np.ndarray) -> np.ndarray:
    return np.where(v > 20.0, v, np.log1p(np.exp(np.minimum(v, 20.0))))


def generate(shape: Shape, seed: int = 0, dt_sigma2: float = 0.5) -> Inputs:
    s = shape
    rng = np.random.default_rng(seed)
    lo, hi = s.dt_bias_range
    x = rng.standard_normal((s.batch, s.seqlen, s.nheads, s.headdim), dtype=np.float32)
    dt_raw = rng.standard_normal((s.batch, s.seqlen, s.nheads), dtype=np.float32)
    u_bias = rng.uniform(math.log(lo), math.log(hi), size=s.nheads)
    u_a = rng.uniform(math.log(1.0), math.log(16.0), size=s.nheads)
    B = rng.standard_normal((s.batch, s.seqlen, s.ngroups, s.dstate), dtype=np.float32)
    C = rng.standard_normal((s.batch, s.seqlen, s.ngroups, s.dstate), dtype=np.float32)
    D = rng.standard_normal(s.nheads).astype(np.float32)
    dy = rng.standard_normal((s.batch, s.seqlen, s.nheads, s.headdim), dtype=np.float32)

    dt_bias = np.log(np.expm1(np.exp(u_bias)))  # inverse softplus of exp(u_bias)
    raw = dt_raw.astype(np.float64) * math.sqrt(dt_sigma2)
    dt = _softplus(raw + dt_bias[None, None, :]).astype(np.float32)
    A = (-np.exp(u_a)).astype(np.float32)
    raw = raw.astype(np.float32)
    bias = dt_bias.astype(np.float32)

    if s.dtype == "bf16":
        x, dt, B, C, dy, raw = (f32_to_bf16_bits(t) for t in (x, dt, B, C, dy, raw))
    elif s.dtype == "fp8":
        x, B, C = (f32_to_e4m3_bits(t) for t in (x, B, C))
        dt, dy, raw = (f32_to_bf16_bits(t) for t in (dt, dy, raw))
    elif s.dtype != "f32":
        raise ValueError(f"unknown dtype {s.dtype!r}")
    return Inputs(s, x, dt, A, B, C, D, dy, raw, bias)


def generate_states(shape: Shape, seed: int = 0):
    """(initial_state, dfinal_state), float32 [batch, nheads, headdim, dstate]."""
    s = shape
    rng = np.random.default_rng([seed, 1])
    dims = (s.batch, s.nheads, s.headdim, s.dstate)
    s0 = rng.standard_normal(dims, dtype=np.float32)
    dfs = rng.standard_normal(dims, dtype=np.float32)
    return s0, dfs


# ---------------------------------------------------------------------------
# Causal depthwise conv1d before the scan.  Its channels are the Mamba-2
# block's conv width nheads*headdim + 2*ngroups*dstate (x, B and C together)
# of each workload; width 4.
CONV_WORKLOADS = {
    name: dict(batch=w["batch"], seqlen=w["seqlen"],
               channels=w["nheads"] * w["headdim"] + 2 * w["ngroups"] * w["dstate"], width=4, dtype=w["dtype"])
    for name, w in WORKLOADS.items()
}


@dataclasses.dataclass
class ConvInputs:
    """x, x_prev, dy in the storage form (uint16 bf16 bits or float32); w, bias float32."""
    x: np.ndarray
    w: np.ndarray
    bias: np.ndarray
    x_prev: np.ndarray
    dy: np.ndarray
    dtype: str

    def as_f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def generate_conv(batch: int, seqlen: int, channels: int, width: int, dtype: str, seed: int = 0) -> ConvInputs:
    """Draw order x ~ N(0,1), w ~ U(-1/sqrt(W), 1/sqrt(W)) (the usual conv
    initialisation for fan-in W), bias likewise, x_prev ~ N(0,1), dy ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, seqlen, channels), dtype=np.float32)
    lim = 1.0 / math.sqrt(width)
    w = rng.uniform(-lim, lim, (channels, width)).astype(np.float32)
    bias = rng.uniform(-lim, lim, channels).astype(np.float32)
    x_prev = rng.standard_normal((batch, width - 1, channels), dtype=np.float32)
    dy = rng.standard_normal((batch, seqlen, channels), dtype=np.float32)
    if dtype == "bf16":
        x, x_prev, dy = (f32_to_bf16_bits(t) for t in (x, x_prev, dy))
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return ConvInputs(x, w, bias, x_prev, dy, dtype)
