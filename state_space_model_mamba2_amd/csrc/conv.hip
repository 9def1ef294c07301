// Causal depthwise conv1d with bias and optional SiLU, the convolution that
// feeds the SSD scan in a Mamba block (the "causal conv" kernel of the LightOn
// page "Training Mamba on AMD GPUs", section "Individual Kernels"):
//   z[b][t][c] = bias[c] + sum_k w[c][k] x[b][t - (W-1) + k][c],  y = act(z)
// token-major [b][L][C]; rows before the sequence come from x_prev
// [b][W-1][C] or are zero.
//
// Bandwidth-bound: every lane owns 4 consecutive channels (one 8-byte bf16
// or 16-byte fp32 vector per row, so a wave reads one contiguous 256/512-byte
// row segment) and walks runs of R tokens, issuing all loads of a run before
// any arithmetic; the W-1 halo rows a run needs come from the neighbouring
// run (L2) or x_prev.  Workgroup: 64 channel vectors x 4 waves; each wave
// takes NR consecutive runs, the 4 waves consecutive run blocks.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"
#include "kernels.h"

namespace ssd {
namespace {

constexpr int kVN = 4;    // channels per lane
constexpr int kNR = 4;    // runs per wave
template <typename T> constexpr int conv_run() { return sizeof(T) == 2 ? 16 : 8; }

__device__ __forceinline__ float sigm(float z) { return 1.0f / (1.0f + __expf(-z)); }

template <typename T>
__device__ __forceinline__ typename Vec4<T>::type zero4() {
  typename Vec4<T>::type v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = from_f<T>(0.0f);
  return v;
}

// Row r (r may be negative: the halo) of sequence b, channels c0..c0+3.
template <typename T>
__device__ __forceinline__ typename Vec4<T>::type load_row(const T* x, const T* prev, int64_t b, int r, int L,
                                                           int C, int c0, int W) {
  typedef typename Vec4<T>::type V4;
  if (r >= 0 && r < L) return *reinterpret_cast<const V4*>(x + ((int64_t)b * L + r) * C + c0);
  if (r < 0 && prev) return *reinterpret_cast<const V4*>(prev + ((int64_t)b * (W - 1) + (r + W - 1)) * C + c0);
  return zero4<T>();
}

template <typename T, int W, bool SILU>
__global__ __launch_bounds__(256) void k_conv_fwd(const T* __restrict__ x, const float* __restrict__ w,
                                                  const float* __restrict__ bias, const T* __restrict__ prev,
                                                  T* __restrict__ y, int L, int C, int rblocks) {
  constexpr int R = conv_run<T>();
  typedef typename Vec4<T>::type V4;
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
    for (int j = 0; j < R + W - 1; ++j) xw[j] = load_row<T>(x, prev, b, t0 - (W - 1) + j, L, C, c0, W);
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
  constexpr int R = conv_run<T>();
  constexpr int NP = kVN * (W + 1);  // partial values per lane: dw taps, then dbias
  typedef typename Vec4<T>::type V4;
  __shared__ float red[4][64][NP + 1];
  const int lane = threadIdx.x & 63;
  const int cv = blockIdx.x * 64 + lane;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.y / rblocks, rb = blockIdx.y % rblocks;
  const bool live = cv * kVN < C;
  const int c0 = live ? cv * kVN : 0;
  float wk[kVN][W], bs[kVN];
#pragma unroll
  for (int e = 0; e < kVN; ++e) {
#pragma unroll
    for (int k = 0; k < W; ++k) wk[e][k] = w[(c0 + e) * W + k];
    bs[e] = bias ? bias[c0 + e] : 0.0f;
  }
  float acc[kVN][W + 1];
#pragma unroll
  for (int e = 0; e < kVN; ++e)
#pragma unroll
    for (int k = 0; k <= W; ++k) acc[e][k] = 0.0f;

  for (int n = 0; n < kNR && live; ++n) {
    const int t0 = ((rb * 4 + wave) * kNR + n) * R;
    if (t0 >= L) break;
    V4 xw[R + 2 * (W - 1)];  // rows t0 - (W-1) .. t0 + R + W - 2
    V4 gw[R + W - 1];        // dy rows t0 .. t0 + R + W - 2, then g
#pragma unroll
    for (int j = 0; j < R + 2 * (W - 1); ++j) xw[j] = load_row<T>(x, prev, b, t0 - (W - 1) + j, L, C, c0, W);
#pragma unroll
    for (int j = 0; j < R + W - 1; ++j) gw[j] = load_row<T>(dy, nullptr, b, t0 + j, L, C, c0, W);
    float g[R + W - 1][kVN];
#pragma unroll
    for (int j = 0; j < R + W - 1; ++j) {
#pragma unroll
      for (int e = 0; e < kVN; ++e) {
        float z = bs[e];
#pragma unroll
        for (int k = 0; k < W; ++k) z += wk[e][k] * to_f(xw[j + k][e]);
        const float d = to_f(gw[j][e]);  // zero past the sequence end
        if (SILU) {
          const float s = sigm(z);
          g[j][e] = d * s * (1.0f + z * (1.0f - s));
        } else {
          g[j][e] = d;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (t0 + i < L) {
        V4 o;
#pragma unroll
        for (int e = 0; e < kVN; ++e) {
          float s = 0.0f;
#pragma unroll
          for (int k = 0; k < W; ++k) s += wk[e][k] * g[i + (W - 1) - k][e];
          o[e] = from_f<T>(s);
#pragma unroll
          for (int k = 0; k < W; ++k) acc[e][k] += g[i][e] * to_f(xw[i + k][e]);
          acc[e][W] += g[i][e];
        }
        *reinterpret_cast<V4*>(dx + ((int64_t)b * L + t0 + i) * C + c0) = o;
      }
    }
    if (t0 == 0 && dprev) {
      // halo row m (time m - (W-1)): sum over taps k <= m of w[k] g[m - k]
#pragma unroll
      for (int m = 0; m < W - 1; ++m) {
        V4 o;
#pragma unroll
        for (int e = 0; e < kVN; ++e) {
          float s = 0.0f;
#pragma unroll
          for (int k = 0; k <= m; ++k) s += wk[e][k] * g[m - k][e];
          o[e] = from_f<T>(s);
        }
        *reinterpret_cast<V4*>(dprev + ((int64_t)b * (W - 1) + m) * C + c0) = o;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < kVN; ++e)
#pragma unroll
    for (int k = 0; k <= W; ++k) red[wave][lane][e * (W + 1) + k] = acc[e][k];
  __syncthreads();
  if (wave == 0 && live) {
    float* o = part + (int64_t)blockIdx.y * C * (W + 1) + (int64_t)c0 * (W + 1);
#pragma unroll
    for (int v = 0; v < NP; ++v) o[v] = (red[0][lane][v] + red[1][lane][v]) + (red[2][lane][v] + red[3][lane][v]);
  }
}

// dw[c][k] and dbias[c]: the workgroup partials summed in a fixed order.
template <int W>
__global__ __launch_bounds__(256) void k_conv_wsum(const float* __restrict__ part, float* __restrict__ dw,
                                                   float* __restrict__ dbias, int C, int nrows) {
  const int v = blockIdx.x * 256 + threadIdx.x;  // c * (W + 1) + k
  if (v >= C * (W + 1)) return;
  float s = 0.0f;
  for (int r = 0; r < nrows; ++r) s += part[(int64_t)r * C * (W + 1) + v];
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
  constexpr int R = conv_run<T>();
  const int rblocks = (int)((a.L + 4 * kNR * R - 1) / (4 * kNR * R));
  const dim3 grid((unsigned)((a.C / kVN + 63) / 64), (unsigned)(a.b * rblocks));
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
  const int64_t R = esz == 2 ? conv_run<bf16>() : conv_run<float>();
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
