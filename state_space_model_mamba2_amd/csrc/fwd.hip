// Forward pass of the SSD chunked scan.
#include "kern_shared.h"

namespace ssd {

// ---------------------------------------------------------------------------
// Chunk scan: for chunk k of head h, rows i in [0, Q):
//   y_i = exp(cs_i) C_i^T Hin_k  +  sum_{j <= i} (C_i . B_j) exp(cs_i - cs_j) dt_j x_j  +  D_h x_i
// One workgroup (4 waves) per (b, k, h).  Output rows are dealt to waves in
// 16-row tiles (zig-zag, so the causal triangle splits evenly).  For each row
// tile a wave
//   1. accumulates C_i . Hin over dstate on the matrix cores and scales rows by exp(cs_i),
//   2. walks source tokens j in steps of 32: reads the precomputed C.B^T
//      accumulator tiles, applies the decay mask exp(cs_i - cs_j) dt_j (zero
//      for j > i) in fp32, and feeds the result straight back as the A
//      fragment of the product with x (chained K mapping), accumulating y,
//   3. adds D x and stores.
// x is staged once per workgroup, transposed (tokens contiguous); the entering
// state Hin_k is staged as [p][n].
template <typename T, int Q, int P, int N>
__global__ __launch_bounds__(256) void k_chunk_scan_fwd(const T* __restrict__ x, const T* __restrict__ dt,
                                                        const float* __restrict__ cs_g, const float* __restrict__ Dp,
                                                        const T* __restrict__ C, const T* __restrict__ hin,
                                                        const T* __restrict__ wt, T* __restrict__ y,
                                                        int L, int H, int G, int K) {
  constexpr int PADQ = 16 / sizeof(T), PADN = 16 / sizeof(T);
  constexpr int NT = Q / 16, TP = P / 16, TILES = NT * (NT + 1) / 2;
  constexpr int NK = (N + 31) / 32;
  __shared__ __attribute__((aligned(16))) T Xt[P][Q + PADQ];
  __shared__ __attribute__((aligned(16))) T Hs[P][N + PADN];
  __shared__ __attribute__((aligned(16))) float cs[Q];
  __shared__ __attribute__((aligned(16))) float dts[Q];

  const int bkh = blockIdx.x;
  const int h = bkh % H, bk = bkh / H, k = bk % K, b = bk / K;
  const int g = h / (H / G);
  const int wave = threadIdx.x / kWave, l = lane_id(), q = l >> 4, c = l & 15;
  const int64_t row0 = (int64_t)b * L + (int64_t)k * Q;

  stage_transposed<T, T, P, 256>(&Xt[0][0], Q + PADQ, x + (row0 * H + h) * P, (int64_t)H * P, Q, nullptr);
  stage_rows<T, T, N, 256>(&Hs[0][0], N + PADN, hin + (int64_t)bkh * P * N, N, P, nullptr);
  const float* csc = cs_g + (((int64_t)b * H + h) * K + k) * Q;
  for (int i = threadIdx.x; i < Q; i += blockDim.x) {
    cs[i] = csc[i];
    dts[i] = to_f(dt[(row0 + i) * H + h]);
  }
  __syncthreads();

  const float Dh = Dp[h];
  const T* wtb = wt + (int64_t)((b * K + k) * G + g) * TILES * 256;

  for (int I = 0; I < NT; ++I) {
    if (zigzag_owner<4>(I) != wave) continue;
    f4 acc[TP];
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) acc[tp] = f4{0.f, 0.f, 0.f, 0.f};

    // 1. state -> output: C_i . Hin (K = dstate)
    const T* crow = C + ((row0 + 16 * I + c) * G + g) * N;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      Frag<T> fa;
      frag_load_k<N>(fa, crow, ks * 32 + 8 * q);
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        Frag<T> fb;
        frag_load_k<N>(fb, &Hs[tp * 16 + c][0], ks * 32 + 8 * q);
        mma(acc[tp], fa, fb);
      }
    }
    {
      const f4 csr = *reinterpret_cast<const f4*>(&cs[16 * I + 4 * q]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __expf(csr[r]);
#pragma unroll
        for (int tp = 0; tp < TP; ++tp) acc[tp][r] *= e;
      }
    }

    // 2. intra-chunk: sum_{j <= i} W_ij exp(cs_i - cs_j) dt_j x_j
    const int ci = 16 * I + c;  // this lane's row i in the W tiles
    const float cs_i = cs[ci];
    for (int J2 = 0; 2 * J2 <= I; ++J2) {
      Frag<T> fa;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int J = 2 * J2 + half;
        const int j0 = 16 * J + 4 * q;
        if (J <= I) {
          const typename Vec4<T>::type wv =
              *reinterpret_cast<const typename Vec4<T>::type*>(wtb + (int64_t)tri_index(I, J) * 256 + l * 4);
          const f4 csj = *reinterpret_cast<const f4*>(&cs[j0]);
          const f4 dtj = *reinterpret_cast<const f4*>(&dts[j0]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float m = (j0 + r <= ci) ? __expf(cs_i - csj[r]) * dtj[r] : 0.0f;
            frag_set<T>(fa, half * 4 + r, to_f(wv[r]) * m);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) frag_set<T>(fa, half * 4 + r, 0.0f);
        }
      }
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        Frag<T> fb;
        frag_load2(fb, &Xt[tp * 16 + c][32 * J2 + 4 * q], &Xt[tp * 16 + c][32 * J2 + 16 + 4 * q]);
        mma(acc[tp], fa, fb);
      }
    }

    // 3. + D x, store rows i = 16I + 4q + r, column p = 16tp + c
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) {
      const int p = tp * 16 + c;
      const typename Vec4<T>::type xv = *reinterpret_cast<const typename Vec4<T>::type*>(&Xt[p][16 * I + 4 * q]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * q + r;
        y[((row0 + i) * H + h) * P + p] = from_f<T>(acc[tp][r] + Dh * to_f(xv[r]));
      }
    }
  }
}

template <typename T, int Q, int P, int N>
void run_fwd(const Layout& lay, const FwdArgs& a, hipStream_t st, const ssd_probe* probe) {
  const int b = (int)lay.b, L = (int)lay.L, H = (int)lay.H, G = (int)lay.G, K = (int)lay.K;
  const T* x = static_cast<const T*>(a.x);
  const T* dt = static_cast<const T*>(a.dt);
  const T* B = static_cast<const T*>(a.B);
  const T* C = static_cast<const T*>(a.C);
  T* hin = static_cast<T*>(a.hin);
  T* wt = static_cast<T*>(a.wt);
  {
    ProbeScope ps(probe, SSD_K_CHUNK_CUMSUM, st);
    k_chunk_cumsum<T, Q><<<dim3(b * H * K), dim3(64), 0, st>>>(dt, a.A, a.cs, L, H, K);
  }
  {
    ProbeScope ps(probe, SSD_K_BMM_FWD, st);
    const int nsplit = 8;
    k_bmm_tiles<T, Q, N, true><<<dim3(b * K * G, nsplit), dim3(256), 0, st>>>(B, C, wt, L, G, K, nsplit);
  }
  {
    ProbeScope ps(probe, SSD_K_CHUNK_STATE, st);
    k_chunk_state<T, Q, P, N, false><<<dim3(b * K * H), dim3(256), 0, st>>>(x, B, dt, a.cs, a.S, L, H, G, K);
  }
  {
    ProbeScope ps(probe, SSD_K_STATE_PASSING, st);
    const int PN = P * N;
    k_state_passing_fwd<T, Q><<<dim3((PN / 4 + 255) / 256, b * H), dim3(256), 0, st>>>(a.S, a.cs, hin, a.final_state, H, K, PN);
  }
  {
    ProbeScope ps(probe, SSD_K_CHUNK_SCAN, st);
    k_chunk_scan_fwd<T, Q, P, N><<<dim3(b * K * H), dim3(256), 0, st>>>(
        x, dt, a.cs, a.D, C, hin, wt, static_cast<T*>(a.y), L, H, G, K);
  }
}

#define SSD_INST_FWD_BF16(Q_, P_, N_) template void run_fwd<bf16, Q_, P_, N_>(const Layout&, const FwdArgs&, hipStream_t, const ssd_probe*);
#define SSD_INST_FWD_F32(Q_, P_, N_) template void run_fwd<float, Q_, P_, N_>(const Layout&, const FwdArgs&, hipStream_t, const ssd_probe*);
SSD_BF16_CONFIGS(SSD_INST_FWD_BF16)
SSD_F32_CONFIGS(SSD_INST_FWD_F32)

}  // namespace ssd
