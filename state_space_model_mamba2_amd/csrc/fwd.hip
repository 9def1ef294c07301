// Forward pass of the SSD chunked scan.
#include "kern_shared.h"

namespace ssd {

// ---------------------------------------------------------------------------
// Chunk scan: for chunk k of head h, rows i in [0, Q):
//   y_i = exp(cs_i) C_i^T Hin_k  +  sum_{j <= i} (C_i . B_j) exp(cs_i - cs_j) dt_j x_j  +  D_h x_i
// One workgroup (4 waves) per (b, k, h).  Output row tiles of 16 tokens are
// dealt to waves in a zig-zag, so the causal triangle splits evenly.  The
// products are formed transposed, y^T = Hin C^T + x^T P^T, so that a lane
// holds 4 consecutive headdim entries of one token (lane (q, c): y[16I + c]
// [16tp + 4q + r]): the row scale exp(cs_i) is one value per lane and the
// stores are 8-byte vectors.  For each row tile a wave
//   1. accumulates Hin . C_i over dstate on the matrix cores and scales by exp(cs_i),
//   2. walks source tokens j in steps of 32: the precomputed C.B^T tiles
//      (forward lane order) times the decay mask exp(cs_i - cs_j) dt_j (zero
//      for j > i) form the B fragment; x^T comes K-major from the staged x
//      rows through the transposing LDS read,
//   3. adds D x and stores.
// x rows of the chunk and the entering state Hin_k are staged once per
// workgroup.  Each wave loads the C rows and all C.B^T tiles of its next row
// tile while it computes the current one.
// Column at which element (r, col) of the staged bf16 x rows is kept: the
// 16-element groups of a row are XOR-permuted by a function of the row, so
// the transposing reads of 4 consecutive rows (and of 8, on 64 banks) meet
// distinct banks without row padding, and 16-byte pieces stay whole.
__device__ __forceinline__ int xcol(int r, int col) { return col ^ (16 * ((r ^ (r >> 2)) & 3)); }

// bf16 with headdim >= 64 keeps x rows unpadded (permuted), which fits three
// workgroups on a CU at chunk 256 / headdim 64 / dstate 128.
template <typename T, typename TI, int Q, int P, int N>
__global__ __launch_bounds__(256, (sizeof(T) == 2 && P % 64 == 0) ? 3 : 2) void k_chunk_scan_fwd(const TI* __restrict__ x, const float* __restrict__ dt,
                                                           const float* __restrict__ cs_g, const float* __restrict__ Dp,
                                                           const TI* __restrict__ C, const T* __restrict__ hin,
                                                           const T* __restrict__ wt, T* __restrict__ y,
                                                           const RowMap rm, int H, int G, int K, int nitems) {
  constexpr int NTH = 256, NW = 4;
  constexpr int NT = Q / 16, TP = P / 16, TILES = NT * (NT + 1) / 2;
  constexpr int NK = (N + 31) / 32, NJ2 = NT / 2;
  constexpr int NSLOT = (NT + NW - 1) / NW;     // row tiles per wave
  constexpr bool XSWZ = sizeof(T) == 2 && P % 64 == 0;
  constexpr int XPITCH = XSWZ ? P : P + 16, HPITCH = N + 16 / sizeof(T);
  constexpr int VN = Vec16<T>::n;
  constexpr int XPIECES = Q * P / VN, HPIECES = P * N / VN;
  constexpr int XPT = (XPIECES + NTH - 1) / NTH, HPT = (HPIECES + NTH - 1) / NTH;
  typedef typename Vec4<T>::type V4;
  typedef typename Vec16<T>::type V;
  __shared__ __attribute__((aligned(16))) T Xs[Q][XPITCH];
  __shared__ __attribute__((aligned(16))) T Hs[P][HPITCH];
  __shared__ __attribute__((aligned(16))) float cs[Q];
  __shared__ __attribute__((aligned(16))) float dts[Q];
  __shared__ __attribute__((aligned(16))) float bfac[Q];  // dt_j exp(cs_r - cs_j), r = last token of j's 32-token step

  const int bkh = xcd_item(blockIdx.x, nitems);
  if (bkh >= nitems) return;  // whole workgroup, before any barrier
  const int h = bkh % H, bk = bkh / H, k = bk % K, b = bk / K;
  const int g = h / (H / G);
  const int wave = threadIdx.x / kWave, l = lane_id(), q = l >> 4, c = l & 15;
  const int64_t row0 = chunk_row0(rm, b, k, Q);
  x = rows_in(rm, k, x, rm.x);
  const float* dtc = dt + (((int64_t)b * H + h) * K + k) * Q;
  C = rows_in(rm, k, C, rm.C);
  y = rows_out(rm, k, y, rm.y);
  const T* wtb = wt + (int64_t)((b * K + k) * G + g) * TILES * 256;

  // row tiles of this wave (zig-zag); NT may be smaller than the wave count
  int Is[NSLOT];
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) Is[sl] = 2 * NW * (sl / 2) + ((sl & 1) ? 2 * NW - 1 - wave : wave);

  // per-row-tile operands: C rows (B operand, K = dstate) and the C.B^T tiles (I, J <= I)
  Frag<T> cf[2][NK];
  V4 wv[2][NT];
  auto tile_load = [&](int set, int I) {
    const TI* crow = C + ((row0 + 16 * I + c) * G + g) * N;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) frag_load_k<N>(cf[set][ks], crow, ks * 32 + 8 * q);
#pragma unroll
    for (int J = 0; J < NT; ++J)  // tiles past the diagonal are never used: load (I, I) instead
      wv[set][J] = *reinterpret_cast<const V4*>(wtb + (int64_t)tri_index(I, J <= I ? J : I) * 256 + l * 4);
  };

  // ---- prologue: all loads first, then LDS stores
  const float* csc = cs_g + (((int64_t)b * H + h) * K + k) * Q;
  constexpr int QPT = (Q + NTH - 1) / NTH;
  float csv[QPT], dtv[QPT];
#pragma unroll
  for (int n = 0; n < QPT; ++n) {
    const int i = threadIdx.x + NTH * n;
    if (Q % NTH == 0 || i < Q) {
      csv[n] = csc[i];
      dtv[n] = dtc[i];
    }
  }
  V xr[XPT], hr[HPT];
#pragma unroll
  for (int n = 0; n < XPT; ++n) {
    const int u = threadIdx.x + NTH * n;
    if (XPIECES % NTH == 0 || u < XPIECES)
      xr[n] = load_vec16<T, TI>(x + ((row0 + u / (P / VN)) * H + h) * P + (u % (P / VN)) * VN);
  }
#pragma unroll
  for (int n = 0; n < HPT; ++n) {
    const int u = threadIdx.x + NTH * n;
    if (HPIECES % NTH == 0 || u < HPIECES) hr[n] = *reinterpret_cast<const V*>(hin + (int64_t)bkh * P * N + u * VN);
  }
  if (Is[0] < NT) tile_load(0, Is[0]);
#pragma unroll
  for (int n = 0; n < QPT; ++n) {
    const int i = threadIdx.x + NTH * n;
    // token r = i | 31 sits in the same wave (32-token steps align with waves)
    const float csr = __shfl(csv[n], (threadIdx.x | 31) & (kWave - 1), kWave);
    if (Q % NTH == 0 || i < Q) {
      cs[i] = csv[n];
      dts[i] = dtv[n];
      bfac[i] = __expf(csr - csv[n]) * dtv[n];
    }
  }
#pragma unroll
  for (int n = 0; n < XPT; ++n) {
    const int u = threadIdx.x + NTH * n;
    if (XPIECES % NTH == 0 || u < XPIECES) {
      const int r = u / (P / VN), col = (u % (P / VN)) * VN;
      *reinterpret_cast<V*>(&Xs[r][XSWZ ? xcol(r, col) : col]) = xr[n];
    }
  }
#pragma unroll
  for (int n = 0; n < HPT; ++n) {
    const int u = threadIdx.x + NTH * n;
    if (HPIECES % NTH == 0 || u < HPIECES) *reinterpret_cast<V*>(&Hs[u / (N / VN)][(u % (N / VN)) * VN]) = hr[n];
  }
  __syncthreads();

  const float Dh = Dp[h];
  // x^T fragment addresses of this lane at source step 0 (rows 4q + c/4 and
  // 16 rows below).  The permutation of row r depends on r only through
  // (r ^ r >> 2) & 3, which for r = 32 J2 + 4q + c/4 is (c/4) ^ q at every
  // step J2, so step J2 reads 32 J2 rows further on: a constant offset.
  int xoff[TP];
#pragma unroll
  for (int tp = 0; tp < TP; ++tp) {
    const int r0 = 4 * q + (c >> 2);
    xoff[tp] = r0 * XPITCH + (XSWZ ? xcol(r0, 16 * tp + 4 * (c & 3)) : 16 * tp + 4 * (c & 3));
  }
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) {
    const int I = Is[sl];
    if (I >= NT) break;
    const int set = sl & 1;
    if (sl + 1 < NSLOT && Is[sl + 1] < NT) tile_load(set ^ 1, Is[sl + 1]);
    f4 acc[TP];
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) acc[tp] = f4{0.f, 0.f, 0.f, 0.f};

    // 1. state -> output: Hin . C_i (K = dstate); lane column i = 16I + c
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        Frag<T> fh;
        frag_load_k<N>(fh, &Hs[16 * tp + c][0], ks * 32 + 8 * q);
        mma(acc[tp], fh, cf[set][ks]);
      }
    }
    const int ci = 16 * I + c;
    const float cs_i = cs[ci];
    {
      const float e = __expf(cs_i);
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) acc[tp] *= e;
    }

    // 2. intra-chunk: sum_{j <= i} W_ij exp(cs_i - cs_j) dt_j x_j.  Steps of 32
    // source tokens wholly before row tile I factor the decay at the step's
    // last token r: exp(cs_i - cs_r) (one per lane) times bfac_j (both <= 1);
    // the step holding the diagonal takes the masked direct form.
#pragma unroll
    for (int J2 = 0; J2 < NJ2; ++J2) {
      if (2 * J2 > I) break;
      Frag<T> fa;                              // P^T as the B operand: col i, K = j (chained)
      if (2 * J2 + 1 < I) {
        const float ai = __expf(cs_i - cs[32 * J2 + 31]);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int J = 2 * J2 + half;
          const f4 bj = *reinterpret_cast<const f4*>(&bfac[16 * J + 4 * q]);
#pragma unroll
          for (int r = 0; r < 4; ++r) frag_set<T>(fa, half * 4 + r, to_f(wv[set][J][r]) * (ai * bj[r]));
        }
      } else {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int J = 2 * J2 + half;
          const int j0 = 16 * J + 4 * q;
          const f4 csj = *reinterpret_cast<const f4*>(&cs[j0]);
          const f4 dtj = *reinterpret_cast<const f4*>(&dts[j0]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float m = (J <= I && j0 + r <= ci) ? __expf(cs_i - csj[r]) * dtj[r] : 0.0f;
            frag_set<T>(fa, half * 4 + r, to_f(wv[set][J][r]) * m);
          }
        }
      }
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        Frag<T> fx;                            // x^T: row p = 16tp + c, K = j (chained)
        if constexpr (XSWZ) {
          const T* a = &Xs[0][0] + 32 * J2 * XPITCH + xoff[tp];  // row r + 16 has row r's permutation
          frag_load_kmajor_at(fx, a, a + 16 * XPITCH);
        } else {
          frag_load_kmajor<32>(fx, &Xs[0][0], XPITCH, 32 * J2, 16 * tp, q, c);
        }
        mma(acc[tp], fx, fa);
      }
    }

    // 3. + D x, store y[i][16tp + 4q + r]
    T* yr = y + ((row0 + ci) * H + h) * P;
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) {
      const V4 xv = *reinterpret_cast<const V4*>(&Xs[ci][XSWZ ? xcol(ci, 16 * tp + 4 * q) : 16 * tp + 4 * q]);
      V4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = from_f<T>(acc[tp][r] + Dh * to_f(xv[r]));
      *reinterpret_cast<V4*>(yr + 16 * tp + 4 * q) = o;
    }
  }
}

template <typename T, typename TI, int Q, int P, int N>
void run_fwd(const Layout& lay, const FwdArgs& a, hipStream_t st, const ssd_probe* probe) {
  const int b = (int)lay.b, H = (int)lay.H, G = (int)lay.G, K = (int)lay.K;
  const TI* x = static_cast<const TI*>(a.x);
  // the cumsum writes the step in float32 (the caller's dt widened, or
  // softplus(dt + dt_bias)); every later kernel reads that
  const float* dt = a.dtf;
  const TI* B = static_cast<const TI*>(a.B);
  const TI* C = static_cast<const TI*>(a.C);
  T* hin = static_cast<T*>(a.hin);
  T* wt = static_cast<T*>(a.wt);
  {
    ProbeScope ps(probe, SSD_K_CUMSUM_BMM, st);
    const int nbkg = b * K * G, nbhk = b * H * K, nbmm = (nbkg + 7) / 8 * 8 * (Q / 64);
    // four adjacent heads per cumsum wave where the head count allows (one 8- or
    // 16-byte load per token instead of four strided ones)
    if (H % 4 == 0)
      k_cumsum_bmm<T, TI, Q, N, 4><<<dim3(nbmm + (nbhk / 4 + 3) / 4), dim3(256), 0, st>>>(
          static_cast<const T*>(a.dt), a.A, a.dt_bias, a.dtf, a.cs, B, C, wt, a.rows, H, G,
          K, a.softplus, nbkg, nbhk);
    else
      k_cumsum_bmm<T, TI, Q, N, 1><<<dim3(nbmm + (nbhk + 3) / 4), dim3(256), 0, st>>>(
          static_cast<const T*>(a.dt), a.A, a.dt_bias, a.dtf, a.cs, B, C, wt, a.rows, H, G,
          K, a.softplus, nbkg, nbhk);
  }
  {
    ProbeScope ps(probe, SSD_K_CHUNK_STATE, st);
    launch_chunk_state<T, TI, TI, Q, P, N, false>(x, B, dt, a.cs, static_cast<T*>(a.S), nullptr, nullptr, a.rows, b, H,
                                                  G, K, st);
  }
  {
    ProbeScope ps(probe, SSD_K_STATE_PASSING, st);
    const int PN = P * N;
    k_state_passing<T, Q, false><<<dim3((PN / 4 + 255) / 256, b * H), dim3(256), 0, st>>>(static_cast<const T*>(a.S), a.cs, a.init, hin, a.final_state, H, K, PN);
  }
  {
    ProbeScope ps(probe, SSD_K_CHUNK_SCAN, st);
    k_chunk_scan_fwd<T, TI, Q, P, N><<<dim3(xcd_grid(b * K * H)), dim3(256), 0, st>>>(
        x, dt, a.cs, a.D, C, hin, wt, static_cast<T*>(a.y), a.rows, H, G, K, b * K * H);
  }
}

#define SSD_INST_FWD_BF16(Q_, P_, N_) template void run_fwd<bf16, bf16, Q_, P_, N_>(const Layout&, const FwdArgs&, hipStream_t, const ssd_probe*);
#define SSD_INST_FWD_FP8(Q_, P_, N_) template void run_fwd<bf16, fp8, Q_, P_, N_>(const Layout&, const FwdArgs&, hipStream_t, const ssd_probe*);
#define SSD_INST_FWD_F32(Q_, P_, N_) template void run_fwd<float, float, Q_, P_, N_>(const Layout&, const FwdArgs&, hipStream_t, const ssd_probe*);
SSD_BF16_CONFIGS(SSD_INST_FWD_BF16)
SSD_BF16_CONFIGS(SSD_INST_FWD_FP8)
SSD_F32_CONFIGS(SSD_INST_FWD_F32)

}  // namespace ssd
