// Causal depthwise conv1d with bias and optional SiLU, the convolution that
// feeds the SSD scan in a Mamba block (the "causal conv" kernel of the LightOn
// page "Training Mamba Models on AMD MI250/MI250X GPUs with Custom Kernels",
// section "Individual Kernels"):
//   z[b][t][c] = bias[c] + sum_k w[c][k] x[b][t - (W-1) + k][c],  y = act(z)
// token-major [b][L][C]; rows before the sequence come from x_prev
// [b][W-1][C] or are zero.
//
// Bandwidth-bound: every lane owns VC consecutive channels (forward 4, one
// 8-byte bf16 or 16-byte fp32 vector per row; backward 2, which keeps its
// larger per-row state within 128+ registers), so a wave reads one contiguous
// row segment, and walks runs of R tokens, issuing all loads of a run before
// any arithmetic; the W-1 halo rows a run needs come from the neighbouring
// run (L2) or x_prev.  Workgroup: 64 channel vectors x 4 waves; each wave
// takes NR consecutive runs, the 4 waves consecutive run blocks.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"
#include "kernels.h"

namespace ssd {
namespace {

constexpr int kVN = 4;    // channels per lane, forward
constexpr int kVB = 2;    // channels per lane, backward
constexpr int kNR = 4;    // runs per wave
template <typename T> constexpr int conv_run() { return sizeof(T) == 2 ? 16 : 8; }       // forward
template <typename T> constexpr int conv_run_bwd() { return 16; }                          // backward

__device__ __forceinline__ float sigm(float z) { return 1.0f / (1.0f + __expf(-z)); }

template <typename T, int VC> struct CVec { typedef T type __attribute__((ext_vector_type(VC))); };

// Row r (r may be negative: the halo) of sequence b, channels c0 .. c0+VC-1;
// zero outside the sequence and the halo.  CLAMP: branch-free, the address is
// clamped to a valid row and the value masked afterwards, so a run's loads
// stay one batch with no wait between them (measured: the backward's 41 row
// loads went from 0.25 to 0.18 ms at the 2.7B conv shape); otherwise each load
// sits in its own branch (the forward's cheaper address arithmetic measured
// 0.093 vs 0.107 ms that way).
template <typename T, int VC, bool CLAMP>
__device__ __forceinline__ typename CVec<T, VC>::type load_row(const T* x, const T* prev, int64_t b, int r, int L,
                                                               int C, int c0, int W) {
  typedef typename CVec<T, VC>::type V;
  if (!CLAMP) {
    if (r >= 0 && r < L) return *reinterpret_cast<const V*>(x + ((int64_t)b * L + r) * C + c0);
    if (r < 0 && prev) return *reinterpret_cast<const V*>(prev + ((int64_t)b * (W - 1) + (r + W - 1)) * C + c0);
    V z;
#pragma unroll
    for (int e = 0; e < VC; ++e) z[e] = from_f<T>(0.0f);
    return z;
  }
  const bool in = r >= 0 && r < L;
  const bool hal = r < 0 && prev != nullptr;
  const int rc = r < 0 ? 0 : (r < L ? r : L - 1);
  const T* p = hal ? prev + ((int64_t)b * (W - 1) + (r + W - 1)) * C + c0 : x + ((int64_t)b * L + rc) * C + c0;
  V v = *reinterpret_cast<const V*>(p);
  const T zero = from_f<T>(0.0f);
#pragma unroll
  for (int e = 0; e < VC; ++e) v[e] = (in || hal) ? v[e] : zero;
  return v;
}

template <typename T, int W, bool SILU>
__global__ __launch_bounds__(256) void k_conv_fwd(const T* __restrict__ x, const float* __restrict__ w,
                                                  const float* __restrict__ bias, const T* __restrict__ prev,
                                                  T* __restrict__ y, int L, int C, int rblocks) {
  constexpr int R = conv_run<T>();
  typedef typename CVec<T, kVN>::type V4;
  const int cv = blockIdx.x * 64 + (threadIdx.x & 63);
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.y / rblocks, rb = blockIdx.y % rblocks;
  if (cv * kVN >= C) return;  // no barrier in this kernel
  const int c0 = cv * kVN;
  float wk[kVN][W], bs[kVN];
#pragma unroll
  for (int e = 0; e < kVN; ++e) {
#pragma unroll
    for (int k = 0; k < W; ++k) wk[e][k] = w[(c0 + e) * W + k];
    bs[e] = bias ? bias[c0 + e] : 0.0f;
  }
  for (int n = 0; n < kNR; ++n) {
    const int t0 = ((rb * 4 + wave) * kNR + n) * R;
    if (t0 >= L) break;
    V4 xw[R + W - 1];  // rows t0 - (W-1) .. t0 + R - 1
#pragma unroll
    for (int j = 0; j < R + W - 1; ++j) xw[j] = load_row<T, kVN, false>(x, prev, b, t0 - (W - 1) + j, L, C, c0, W);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (t0 + i < L) {
        V4 o;
#pragma unroll
        for (int e = 0; e < kVN; ++e) {
          float z = bs[e];
#pragma unroll
          for (int k = 0; k < W; ++k) z += wk[e][k] * to_f(xw[i + k][e]);
          o[e] = from_f<T>(SILU ? z * sigm(z) : z);
        }
        *reinterpret_cast<V4*>(y + ((int64_t)b * L + t0 + i) * C + c0) = o;
      }
    }
  }
}

// Backward: per run, g = dy * act'(z) for rows t0 .. t0 + R + W - 2 (z
// recomputed from x), dx[s] = sum_k w[k] g[s + W-1 - k] for the run's rows,
// the run's rows' contributions to dw and dbias, and for the first run of a
// sequence the halo's gradient dx_prev.  dw / dbias partials: the 4 waves of
// a workgroup are summed in LDS, one partial row per workgroup.
template <typename T, int W, bool SILU>
__global__ __launch_bounds__(256) void k_conv_bwd(const T* __restrict__ x, const float* __restrict__ w,
                                                  const float* __restrict__ bias, const T* __restrict__ prev,
                                                  const T* __restrict__ dy, T* __restrict__ dx,
                                                  T* __restrict__ dprev, float* __restrict__ part, int L, int C,
                                                  int rblocks) {
  constexpr int R = conv_run_bwd<T>();
  constexpr int NP = kVB * (W + 1);  // partial values per lane: dw taps, then dbias
  typedef typename CVec<T, kVB>::type V4;
  __shared__ float red[4][64][NP + 1];
  const int lane = threadIdx.x & 63;
  const int cv = blockIdx.x * 64 + lane;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.y / rblocks, rb = blockIdx.y % rblocks;
  const bool live = cv * kVB < C;
  const int c0 = live ? cv * kVB : 0;
  float wk[kVB][W], bs[kVB];
#pragma unroll
  for (int e = 0; e < kVB; ++e) {
#pragma unroll
    for (int k = 0; k < W; ++k) wk[e][k] = w[(c0 + e) * W + k];
    bs[e] = bias ? bias[c0 + e] : 0.0f;
  }
  float acc[kVB][W + 1];
#pragma unroll
  for (int e = 0; e < kVB; ++e)
#pragma unroll
    for (int k = 0; k <= W; ++k) acc[e][k] = 0.0f;

  for (int n = 0; n < kNR && live; ++n) {
    const int t0 = ((rb * 4 + wave) * kNR + n) * R;
    if (t0 >= L) break;
    V4 xw[R + 2 * (W - 1)];  // rows t0 - (W-1) .. t0 + R + W - 2
    V4 gw[R + W - 1];        // dy rows t0 .. t0 + R + W - 2
#pragma unroll
    for (int j = 0; j < R + 2 * (W - 1); ++j) xw[j] = load_row<T, kVB, true>(x, prev, b, t0 - (W - 1) + j, L, C, c0, W);
#pragma unroll
    for (int j = 0; j < R + W - 1; ++j) gw[j] = load_row<T, kVB, true>(dy, nullptr, b, t0 + j, L, C, c0, W);
    // one pass over rows t = t0 + j: g of the row, its dw / dbias terms (the
    // run's own rows), and, once the window holds g of rows s .. s + W - 1,
    // dx of row s = t - (W-1) (the halo row for s < 0 in the first run).
    float gwin[W][kVB];  // g of rows t - (W-1) .. t; rows before the run count as zero
#pragma unroll
    for (int m = 0; m < W; ++m)
#pragma unroll
      for (int e = 0; e < kVB; ++e) gwin[m][e] = 0.0f;
#pragma unroll
    for (int j = 0; j < R + W - 1; ++j) {
#pragma unroll
      for (int e = 0; e < kVB; ++e) {
        float z = bs[e];
#pragma unroll
        for (int k = 0; k < W; ++k) z += wk[e][k] * to_f(xw[j + k][e]);
        const float d = to_f(gw[j][e]);  // zero past the sequence end
        float gj = d;
        if (SILU) {
          const float sg = sigm(z);
          gj = d * sg * (1.0f + z * (1.0f - sg));
        }
#pragma unroll
        for (int m = 0; m < W - 1; ++m) gwin[m][e] = gwin[m + 1][e];
        gwin[W - 1][e] = gj;
        if (j < R) {
#pragma unroll
          for (int k = 0; k < W; ++k) acc[e][k] += gj * to_f(xw[j + k][e]);
          acc[e][W] += gj;
        }
      }
      const int i = j - (W - 1);  // row s = t0 + i gets its dx now
      const bool own = i >= 0 && i < R && t0 + i < L;
      const bool halo = i < 0 && t0 == 0 && dprev != nullptr;
      if (own || halo) {
        V4 o;
#pragma unroll
        for (int e = 0; e < kVB; ++e) {
          float sx = 0.0f;
#pragma unroll
          for (int k = 0; k < W; ++k) sx += wk[e][k] * gwin[W - 1 - k][e];
          o[e] = from_f<T>(sx);
        }
        T* dst = own ? dx + ((int64_t)b * L + t0 + i) * C + c0 : dprev + ((int64_t)b * (W - 1) + j) * C + c0;
        *reinterpret_cast<V4*>(dst) = o;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < kVB; ++e)
#pragma unroll
    for (int k = 0; k <= W; ++k) red[wave][lane][e * (W + 1) + k] = acc[e][k];
  __syncthreads();
  if (wave == 0 && live) {
    float* o = part + (int64_t)blockIdx.y * C * (W + 1) + (int64_t)c0 * (W + 1);
#pragma unroll
    for (int v = 0; v < NP; ++v) o[v] = (red[0][lane][v] + red[1][lane][v]) + (red[2][lane][v] + red[3][lane][v]);
  }
}

// dw[c][k] and dbias[c]: the workgroup partials summed in a fixed order
// (eight interleaved running sums, so eight loads are in flight, then a
// fixed tree).
template <int W>
__global__ __launch_bounds__(256) void k_conv_wsum(const float* __restrict__ part, float* __restrict__ dw,
                                                   float* __restrict__ dbias, int C, int nrows) {
  const int v = blockIdx.x * 256 + threadIdx.x;  // c * (W + 1) + k
  if (v >= C * (W + 1)) return;
  const int64_t rs = (int64_t)C * (W + 1);
  float p[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int r = 0;
  for (; r + 8 <= nrows; r += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) p[u] += part[(r + u) * rs + v];
  }
  for (int u = 0; r < nrows; ++r, ++u) p[u] += part[r * rs + v];
  const float s = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  const int c = v / (W + 1), k = v % (W + 1);
  if (k < W) dw[c * W + k] = s;
  else if (dbias) dbias[c] = s;
}

template <typename T, int W>
void launch_fwd(const ConvArgs& a, hipStream_t st) {
  constexpr int R = conv_run<T>();
  const int rblocks = (int)((a.L + 4 * kNR * R - 1) / (4 * kNR * R));
  const dim3 grid((unsigned)((a.C / kVN + 63) / 64), (unsigned)(a.b * rblocks));
  const T* x = static_cast<const T*>(a.x);
  const T* prev = static_cast<const T*>(a.x_prev);
  T* y = static_cast<T*>(a.y);
  if (a.silu) k_conv_fwd<T, W, true><<<grid, dim3(256), 0, st>>>(x, a.w, a.bias, prev, y, (int)a.L, (int)a.C, rblocks);
  else k_conv_fwd<T, W, false><<<grid, dim3(256), 0, st>>>(x, a.w, a.bias, prev, y, (int)a.L, (int)a.C, rblocks);
}

template <typename T, int W>
void launch_bwd(const ConvArgs& a, hipStream_t st) {
  constexpr int R = conv_run_bwd<T>();
  const int rblocks = (int)((a.L + 4 * kNR * R - 1) / (4 * kNR * R));
  const dim3 grid((unsigned)((a.C / kVB + 63) / 64), (unsigned)(a.b * rblocks));
  const T* x = static_cast<const T*>(a.x);
  const T* prev = static_cast<const T*>(a.x_prev);
  const T* dy = static_cast<const T*>(a.dy);
  T* dx = static_cast<T*>(a.dx);
  T* dprev = static_cast<T*>(a.dx_prev);
  if (a.silu)
    k_conv_bwd<T, W, true><<<grid, dim3(256), 0, st>>>(x, a.w, a.bias, prev, dy, dx, dprev, a.part, (int)a.L,
                                                       (int)a.C, rblocks);
  else
    k_conv_bwd<T, W, false><<<grid, dim3(256), 0, st>>>(x, a.w, a.bias, prev, dy, dx, dprev, a.part, (int)a.L,
                                                        (int)a.C, rblocks);
  const int nv = (int)(a.C * (W + 1));
  k_conv_wsum<W><<<dim3((unsigned)((nv + 255) / 256)), dim3(256), 0, st>>>(a.part, a.dw, a.dbias, (int)a.C,
                                                                           (int)(a.b * rblocks));
}

template <typename T>
void dispatch(bool fwd, const ConvArgs& a, hipStream_t st) {
  switch (a.W) {
    case 2: fwd ? launch_fwd<T, 2>(a, st) : launch_bwd<T, 2>(a, st); break;
    case 3: fwd ? launch_fwd<T, 3>(a, st) : launch_bwd<T, 3>(a, st); break;
    default: fwd ? launch_fwd<T, 4>(a, st) : launch_bwd<T, 4>(a, st); break;
  }
}

}  // namespace

int64_t conv_partial_rows(int64_t b, int64_t L, int esz) {
  const int64_t R = esz == 2 ? conv_run_bwd<bf16>() : conv_run_bwd<float>();
  return b * ((L + 4 * kNR * R - 1) / (4 * kNR * R));
}

void run_conv_fwd(const ConvArgs& a, hipStream_t st) {
  if (a.esz == 2) dispatch<bf16>(true, a, st);
  else dispatch<float>(true, a, st);
}

void run_conv_bwd(const ConvArgs& a, hipStream_t st) {
  if (a.esz == 2) dispatch<bf16>(false, a, st);
  else dispatch<float>(false, a, st);
}

}  // namespace ssd
