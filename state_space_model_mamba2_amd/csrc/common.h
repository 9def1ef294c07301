// Shared device helpers for the SSD kernels (gfx950 / CDNA4, wave64).
//
// Matrix-core conventions used by every kernel
// --------------------------------------------
// All products go through 16x16 output tiles of v_mfma_f32_16x16x32_bf16
// (bf16 operands) or eight chained v_mfma_f32_16x16x4_f32 (fp32 operands).
// A "fragment" is the 8 K-values one lane contributes to a 16x16x32 step:
//   A fragment : row  m = lane % 16 of the A tile,  K-slots s = 0..7
//   B fragment : col  n = lane % 16 of the B tile,  K-slots s = 0..7
// Lane group q = lane / 16 and slot s together name one logical k.  The sum
// over k does not care which logical k sits in which (q, s) as long as the A
// and B fragments agree, so two mappings are used:
//   contiguous : k = 8q + s                         (one 16-byte load in bf16)
//   chained    : k = 4q + s (s < 4), 16 + 4q + s-4   (matches the rows a lane
//                holds in a 16x16 accumulator, so an accumulator tile pair can
//                be fed straight back in as the next product's A/B fragment)
// Accumulator tile: lane holds col n = lane % 16, rows m = 4q + r, r = 0..3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16;

constexpr int kWave = 64;

// ---- scalar conversions ---------------------------------------------------
__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return (bf16)v; }

// 16-byte vector of T: 8 bf16 or 4 floats.
template <typename T> struct Vec16;
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int n = 8; };
template <> struct Vec16<float> { typedef f4 type; static constexpr int n = 4; };

// ---- FP8 (OCP E4M3: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
// no infinities, S.1111.111 is NaN) ----------------------------------------
typedef unsigned char fp8;

// Eight codes (little-endian bytes of w) widened to bf16, exactly: every E4M3
// value is a bf16 value.  gfx950's packed conversion with scale 1 widens two
// codes (bytes 0-1, or 2-3 with the high selector) in element order; checked
// on the GPU against the exact value of all 256 codes (NaN stays NaN, -0 is
// kept).  A bit-manipulation widening cost ten ALU operations per code and
// made the FP8 forward slower than bf16.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint2 w) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true);
  typedef __bf16 bf16x4l __attribute__((ext_vector_type(4)));
  const bf16x4l lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const bf16x4l hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// One 16-byte vector of compute type T from 8 (bf16) or 4 (fp32) elements of
// storage type TI at p: a plain load, or eight FP8 codes widened to bf16.
template <typename T, typename TI>
__device__ __forceinline__ typename Vec16<T>::type load_vec16(const TI* p);
template <>
__device__ __forceinline__ bf16x8 load_vec16<bf16, bf16>(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
template <>
__device__ __forceinline__ f4 load_vec16<float, float>(const float* p) { return *reinterpret_cast<const f4*>(p); }
template <>
__device__ __forceinline__ bf16x8 load_vec16<bf16, fp8>(const fp8* p) {
  return e4m3x8_to_bf16(*reinterpret_cast<const uint2*>(p));
}

// ---- fragments --------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ void mma(f4& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f4& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], c, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ void frag_set(Frag<T>& f, int s, float v);
template <> __device__ __forceinline__ void frag_set<bf16>(Frag<bf16>& f, int s, float v) { f.v[s] = (bf16)v; }
template <> __device__ __forceinline__ void frag_set<float>(Frag<float>& f, int s, float v) { f.v[s] = v; }
template <typename T> __device__ __forceinline__ float frag_get(const Frag<T>& f, int s) { return (float)f.v[s]; }

// 8 contiguous elements (16-byte aligned for bf16, 32-byte pair for fp32;
// eight FP8 codes, 8-byte aligned, are widened to a bf16 fragment).
__device__ __forceinline__ void frag_load(Frag<bf16>& f, const bf16* p) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void frag_load(Frag<bf16>& f, const fp8* p) {
  f.v = e4m3x8_to_bf16(*reinterpret_cast<const uint2*>(p));
}
__device__ __forceinline__ void frag_load(Frag<float>& f, const float* p) {
  f4 a = *reinterpret_cast<const f4*>(p);
  f4 b = *reinterpret_cast<const f4*>(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
// Two runs of 4 contiguous elements (chained mapping).
__device__ __forceinline__ void frag_load2(Frag<bf16>& f, const bf16* p0, const bf16* p1) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void frag_load2(Frag<float>& f, const float* p0, const float* p1) {
  f4 a = *reinterpret_cast<const f4*>(p0);
  f4 b = *reinterpret_cast<const f4*>(p1);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// Fragment whose K runs down the rows of a row-major LDS tile ("K-major"):
// lane (q, c) receives tile[k0 + kc(q, s)][col0 + c] for the chained K
// mapping kc(q, s) = 4q + s (s < 4), 16 + 4q + s - 4 (s >= 4).  With
// KD = 16 the second run (rows k0 + 16 ..) is zero and never read.
// bf16 uses the gfx950 transposing LDS read ds_read_b64_tr_b16: in each
// group of 16 lanes, lane l supplies the address of 4 consecutive values
// (row k0 + 4q + l/4, columns col0 + 4(l%4) ..) and receives column col0 + l
// of the group's 4 rows.  Rows must be 8-byte aligned; a row pitch of 8
// (mod 16) dwords keeps the 16 rows of one read on distinct banks.
// fp32 has no transposing read and takes eight scalar reads.
template <int KD>
__device__ __forceinline__ void frag_load_kmajor(Frag<bf16>& f, const bf16* tile, int pitch, int k0, int col0, int q,
                                                 int c) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s* lds_v4s;
  const bf16* a0 = tile + (k0 + 4 * q + (c >> 2)) * pitch + col0 + 4 * (c & 3);
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(a0));
  v4s hi = {0, 0, 0, 0};
  if constexpr (KD % 32 == 0) hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(a0 + 16 * pitch));
  f.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// The same transposing read from per-lane addresses of the two 16-row runs
// (for tiles stored in a permuted layout): lane (q, c) passes the address of
// its 4 values in rows k0 + 4q + c/4 and k0 + 16 + 4q + c/4.
__device__ __forceinline__ void frag_load_kmajor_at(Frag<bf16>& f, const bf16* lo_addr, const bf16* hi_addr) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s* lds_v4s;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(lo_addr));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(hi_addr));
  f.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
template <int KD>
__device__ __forceinline__ void frag_load_kmajor(Frag<float>& f, const float* tile, int pitch, int k0, int col0,
                                                 int q, int c) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int k = s < 4 ? 4 * q + s : 16 + 4 * q + s - 4;
    f.v[s] = (KD % 32 == 0 || s < 4) ? tile[(k0 + k) * pitch + col0 + c] : 0.0f;
  }
}

// 16 bytes per lane from global memory straight into LDS (gfx950
// global_load_lds_dwordx4): lane l's bytes land at lds_wave_base + 16 l, where
// lds_wave_base is the same for the whole wave (checked on gfx950 with an
// in-bounds probe).  Counted by vmcnt like any vector-memory load; the caller
// waits for it (s_waitcnt vmcnt) before a barrier that publishes the data.
// s_waitcnt immediate for vmcnt(n) lgkmcnt(0) (expcnt not waited for):
// vmcnt's low four bits at [3:0], its high two at [15:14].
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }
// vmcnt(n) alone (lgkmcnt field at its maximum, 15).  Vector-memory loads,
// copies into LDS and stores leave this counter in the order they were
// issued; the compiler assumes no such order between copies into LDS and
// loads into registers and, with both in flight, waits for vmcnt(0) before
// a register's first use.  A kernel that keeps copies in flight over such a
// use waits for the register itself with this count (everything issued
// after it) before that use.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
// lgkmcnt(0) alone (vmcnt and expcnt fields at their maxima): LDS stores
// written in asm, which the compiler does not count, have completed.
constexpr int kWaitLgkm0 = 0xC07F;

__device__ __forceinline__ void lds_copy16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// ---- LDS staging --------------------------------------------------------------
// 4 consecutive storage elements (one lane's share of an accumulator tile).
template <typename T> struct Vec4;
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef f4 type; };

// Copy `rows` x COLS of a global tile (COLS contiguous, row stride gstride
// source elements) into LDS transposed, converting to TD:
//   dst[c * dpitch + r] = src[r][c] * scale[r]          (scale may be null)
// Work unit: 4 rows x one 16-byte column vector, written as 4-row runs.
// rows must be a multiple of 4.
template <typename TD, typename TS, int COLS, int NTHREADS>
__device__ __forceinline__ void stage_transposed(TD* __restrict__ dst, int dpitch, const TS* __restrict__ src,
                                                 int64_t gstride, int rows, const float* __restrict__ scale) {
  constexpr int VN = Vec16<TS>::n;
  constexpr int CU = COLS / VN;
  typedef typename Vec16<TS>::type V;
  const int units = (rows / 4) * CU;
  for (int u = threadIdx.x; u < units; u += NTHREADS) {
    const int cu = u % CU, r0 = (u / CU) * 4, c0 = cu * VN;
    V v[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) v[rr] = *reinterpret_cast<const V*>(src + (int64_t)(r0 + rr) * gstride + c0);
    float sc[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sc[rr] = scale ? scale[r0 + rr] : 1.0f;
#pragma unroll
    for (int e = 0; e < VN; ++e) {
      typename Vec4<TD>::type w;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) w[rr] = from_f<TD>(to_f(v[rr][e]) * sc[rr]);
      *reinterpret_cast<typename Vec4<TD>::type*>(dst + (c0 + e) * dpitch + r0) = w;
    }
  }
}

// Copy `rows` x COLS into LDS without transposing, converting to TD:
//   dst[r * dpitch + c] = src[r][c] * scale[r]          (scale may be null)
template <typename TD, typename TS, int COLS, int NTHREADS>
__device__ __forceinline__ void stage_rows(TD* __restrict__ dst, int dpitch, const TS* __restrict__ src,
                                           int64_t gstride, int rows, const float* __restrict__ scale) {
  constexpr int VN = Vec16<TS>::n;
  constexpr int CU = COLS / VN;
  typedef typename Vec16<TS>::type V;
  const int units = rows * CU;
  for (int u = threadIdx.x; u < units; u += NTHREADS) {
    const int cu = u % CU, r = u / CU;
    const V v = *reinterpret_cast<const V*>(src + (int64_t)r * gstride + cu * VN);
    const float sc = scale ? scale[r] : 1.0f;
    TD* d = dst + r * dpitch + cu * VN;
    if constexpr (sizeof(TD) == sizeof(TS) && VN == 8) {
      if (!scale) { *reinterpret_cast<V*>(d) = v; continue; }
    }
    if constexpr (sizeof(TD) == sizeof(TS) && VN == 4) {
      if (!scale) { *reinterpret_cast<V*>(d) = v; continue; }
    }
#pragma unroll
    for (int e0 = 0; e0 < VN; e0 += 4) {
      typename Vec4<TD>::type w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = from_f<TD>(to_f(v[e0 + e]) * sc);
      *reinterpret_cast<typename Vec4<TD>::type*>(d + e0) = w;
    }
  }
}

// ---- XCD-aware work mapping ------------------------------------------------------
// Workgroups are dispatched round-robin over the chip's 8 XCDs (workgroup i
// on XCD i % 8), and each XCD has its own L2.  Workgroup i takes item
// (i % 8) * ceil(n / 8) + i / 8, so each XCD walks one contiguous run of
// items in order: consecutive items (the heads of one chunk, which read that
// chunk's B / C rows and C.B^T tiles) share one L2 instead of fetching the
// shared rows into all eight.  The grid is xcd_grid(n) workgroups; the
// mapped index is >= n for the padding workgroups of the last run.
constexpr int kXcds = 8;
__host__ __device__ constexpr int xcd_grid(int n) { return (n + kXcds - 1) / kXcds * kXcds; }
__device__ __forceinline__ int xcd_item(int bid, int n) { return (bid % kXcds) * ((n + kXcds - 1) / kXcds) + bid / kXcds; }

// ---- wave-level scans and reductions (wave64) -------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Inclusive prefix sum across the 64 lanes.
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    float o = __shfl_up(v, off, kWave);
    if (l >= off) v += o;
  }
  return v;
}
// Inclusive suffix sum across the 64 lanes (lane l gets sum over lanes >= l).
__device__ __forceinline__ float wave_inclusive_suffix(float v) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    float o = __shfl_down(v, off, kWave);
    if (l + off < kWave) v += o;
  }
  return v;
}
// Register-only lane move inside each row of 16 lanes (a DPP operand).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Eight sums over each row of 16 lanes at once: every value v[0..7] is
// summed over the 16 lanes of the row, and lane c keeps the total of value
// 4 b3 + 2 b2 + b1 (b3, b2, b1 = bits 3, 2, 1 of c; lanes c and c ^ 1 hold the
// same total).  A butterfly over the lane partners c ^ 15, c ^ 7, c ^ 3, c ^ 1
// (row mirror, half-row mirror, two quad permutations) in which each exchange
// halves the values a lane keeps: the lane whose bit is set keeps the upper
// half and sends the lower, its partner the reverse, so 7 exchanges do the
// work of 8 separate 4-step row sums.
__device__ __forceinline__ float sum16_spread8(const float (&v)[8]) {
  const int c = threadIdx.x & 15;
  const bool b3 = c & 8, b2 = c & 4, b1 = c & 2;
  float w[4], z[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = (b3 ? v[k + 4] : v[k]) + dpp_mov<0x140>(b3 ? v[k] : v[k + 4]);
#pragma unroll
  for (int k = 0; k < 2; ++k) z[k] = (b2 ? w[k + 2] : w[k]) + dpp_mov<0x141>(b2 ? w[k] : w[k + 2]);
  float u = (b1 ? z[1] : z[0]) + dpp_mov<0x1B>(b1 ? z[0] : z[1]);  // quad_perm [3, 2, 1, 0]
  u += dpp_mov<0xB1>(u);                                             // quad_perm [1, 0, 3, 2]
  return u;
}
// Sum over the 4 lanes sharing lane % 16 (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float sum_q(float v) {
  v += __shfl_xor(v, 16, kWave);
  v += __shfl_xor(v, 32, kWave);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Balanced ownership of 16-row tiles across NW waves: tiles are dealt in a
// zig-zag (0..NW-1, NW-1..0, ...) so triangular work evens out.
template <int NW>
__device__ __forceinline__ int zigzag_owner(int tile) {
  const int m = tile % (2 * NW);
  return m < NW ? m : 2 * NW - 1 - m;
}

}  // namespace ssd
