// Backward pass of the SSD chunked scan.
#include "kern_shared.h"

namespace ssd {

// ---------------------------------------------------------------------------
// Per-head chunk backward: one workgroup (4 waves) per (b, k, h).
// With Gk = dL/d(state leaving chunk k), xt_j = dt_j x_j, W_ij = C_i . B_j,
// Lam_ij = exp(cs_i - cs_j) (j <= i) and P = W o Lam:
//   dxt_j = e_j B_j^T Gk + sum_{i >= j} P_ij dy_i,        e_j = exp(cs_{Q-1} - cs_j)
//   R_ij  = <dy_i, xt_j> P_ij
//   dcs_i = sum_j R_ij - sum_i' R_i'i + exp(cs_i) <dy_i, Hin_k^T C_i> - q_i,
//           q_j = <xt_j, e_j B_j^T Gk>;   dcs_{Q-1} += sum_j q_j + exp(cs_{Q-1}) <Gk, Hin_k>
//   dl    = reverse cumsum of dcs inside the chunk
//   ddt_j = A dl_j + <dxt_j, x_j>,  dx_j = dt_j dxt_j + D dy_j
// plus the chunk's partial sums of dA (sum_j dt_j dl_j) and dD (sum <dy, x>).
// Each (row tile I, column tile J) pair is formed twice on the matrix cores:
// as R (lanes own a column j; its rows are summed in-lane for the column sums
// and it feeds dxt) and as R^T (lanes own a row i; summed in-lane for the row
// sums).  Both come from the same operands and from C.B^T tiles holding
// identical values in the two lane orders, so the row and column sums cancel
// exactly where the exact gradient cancels.  Row tiles and column tiles are
// dealt to waves in zig-zag order; per-wave partial row sums are added in a
// fixed order.
template <typename T, int Q, int P, int N>
__global__ __launch_bounds__(256) void k_chunk_scan_bwd(
    const T* __restrict__ x, const T* __restrict__ dt, const float* __restrict__ cs_g, const float* __restrict__ Ap,
    const float* __restrict__ Dp, const T* __restrict__ B, const T* __restrict__ C, const T* __restrict__ hin,
    const T* __restrict__ gst, const T* __restrict__ wf, const T* __restrict__ wb, const T* __restrict__ dy,
    T* __restrict__ dx, T* __restrict__ ddt, float* __restrict__ dapart, float* __restrict__ ddpart,
    int L, int H, int G, int K) {
  constexpr int NW = 4, NTH = NW * kWave;
  constexpr int PADQ = 16 / sizeof(T), PADN = 16 / sizeof(T);
  constexpr int NT = Q / 16, TP = P / 16, TILES = NT * (NT + 1) / 2;
  constexpr int NK = (N + 31) / 32, NKP = (P + 31) / 32;
  constexpr int TPL = Q / kWave;
  typedef typename Vec4<T>::type V4;
  __shared__ __attribute__((aligned(16))) T DYt[P][Q + PADQ];
  __shared__ __attribute__((aligned(16))) T Xt[P][Q + PADQ];
  __shared__ __attribute__((aligned(16))) T Hs[P][N + PADN];
  __shared__ __attribute__((aligned(16))) T Gs[P][N + PADN];
  __shared__ __attribute__((aligned(16))) float cs[Q];
  __shared__ __attribute__((aligned(16))) float dts[Q];
  __shared__ float rowacc[NW][Q];
  __shared__ float colacc[Q];
  __shared__ float qv[Q];
  __shared__ float ddtd[Q];
  __shared__ float red[2 * NW];

  const int bkh = blockIdx.x;
  const int h = bkh % H, bk = bkh / H, k = bk % K, b = bk / K;
  const int g = h / (H / G);
  const int wave = threadIdx.x / kWave, l = lane_id(), q = l >> 4, c = l & 15;
  const int64_t row0 = (int64_t)b * L + (int64_t)k * Q;

  stage_transposed<T, T, P, NTH>(&DYt[0][0], Q + PADQ, dy + (row0 * H + h) * P, (int64_t)H * P, Q, nullptr);
  stage_transposed<T, T, P, NTH>(&Xt[0][0], Q + PADQ, x + (row0 * H + h) * P, (int64_t)H * P, Q, nullptr);
  stage_rows<T, T, N, NTH>(&Hs[0][0], N + PADN, hin + (int64_t)bkh * P * N, N, P, nullptr);
  stage_rows<T, T, N, NTH>(&Gs[0][0], N + PADN, gst + (int64_t)bkh * P * N, N, P, nullptr);
  const float* csc = cs_g + (((int64_t)b * H + h) * K + k) * Q;
  for (int i = threadIdx.x; i < Q; i += NTH) {
    cs[i] = csc[i];
    dts[i] = to_f(dt[(row0 + i) * H + h]);
#pragma unroll
    for (int w = 0; w < NW; ++w) rowacc[w][i] = 0.0f;
  }
  __syncthreads();

  const float cs_last = cs[Q - 1];
  const float Dh = Dp[h];
  const int64_t tbase = (int64_t)((b * K + k) * G + g) * TILES * 256;
  const T* wfb = wf + tbase;
  const T* wbb = wb + tbase;

  // (1) state -> output part of dcs: exp(cs_i) <dy_i, Hin^T C_i> for owned row tiles.
  for (int I = 0; I < NT; ++I) {
    if (zigzag_owner<NW>(I) != wave) continue;
    f4 acc[TP];
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) acc[tp] = f4{0.f, 0.f, 0.f, 0.f};
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
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) {
      const V4 dv = *reinterpret_cast<const V4*>(&DYt[tp * 16 + c][16 * I + 4 * q]);
#pragma unroll
      for (int r = 0; r < 4; ++r) part[r] += acc[tp][r] * to_f(dv[r]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * I + 4 * q + r;
      const float s = sum16(part[r]) * __expf(cs[i]);
      if (c == 0) rowacc[wave][i] += s;
    }
  }

  // (2) owned column tiles J: dxt, q, row and column sums of R, ddt (direct part), dx.
  float rowpart[NT];  // this lane's partial row sums, row i = 16 I + c
#pragma unroll
  for (int I = 0; I < NT; ++I) rowpart[I] = 0.0f;
  for (int J = 0; J < NT; ++J) {
    if (zigzag_owner<NW>(J) != wave) continue;
    f4 adx[TP];
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) adx[tp] = f4{0.f, 0.f, 0.f, 0.f};
    // state part: B_j^T Gk (K = dstate), scaled by e_j
    const T* brow = B + ((row0 + 16 * J + c) * G + g) * N;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      Frag<T> fa;
      frag_load_k<N>(fa, brow, ks * 32 + 8 * q);
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        Frag<T> fb;
        frag_load_k<N>(fb, &Gs[tp * 16 + c][0], ks * 32 + 8 * q);
        mma(adx[tp], fa, fb);
      }
    }
    {
      const f4 csr = *reinterpret_cast<const f4*>(&cs[16 * J + 4 * q]);
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        const V4 xv = *reinterpret_cast<const V4*>(&Xt[tp * 16 + c][16 * J + 4 * q]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          adx[tp][r] *= __expf(cs_last - csr[r]);
          part[r] += adx[tp][r] * to_f(xv[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * J + 4 * q + r;
        const float s = sum16(part[r]) * dts[j];
        if (c == 0) qv[j] = s;
      }
    }
    // intra part: row tiles I >= J, two per step (32 tokens i); both tiles'
    // operands (C.B^T tiles in both lane orders, dy fragments) are requested
    // before either is used.
    const int cj = 16 * J + c;  // this lane's column j in R
    const float cs_cj = cs[cj], dt_cj = dts[cj];
    const int rj0 = 16 * J + 4 * q;  // this lane's rows j in R^T
    const f4 cs_rj = *reinterpret_cast<const f4*>(&cs[rj0]);
    const f4 dt_rj = *reinterpret_cast<const f4*>(&dts[rj0]);
    Frag<T> xf[NKP];
    const T* xrow = x + ((row0 + cj) * H + h) * P;
#pragma unroll
    for (int kp = 0; kp < NKP; ++kp) frag_load_k<P>(xf[kp], xrow, kp * 32 + 8 * q);
    float colsum = 0.0f;
#pragma unroll
    for (int I2 = 0; I2 < NT / 2; ++I2) {
      if (2 * I2 + 1 < J) continue;
      V4 wv[2], wtv[2];
      Frag<T> fd[2][NKP];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int I = 2 * I2 + half;
        if (I >= J) {
          wv[half] = *reinterpret_cast<const V4*>(wbb + (int64_t)tri_index(I, J) * 256 + l * 4);
          wtv[half] = *reinterpret_cast<const V4*>(wfb + (int64_t)tri_index(I, J) * 256 + l * 4);
          const T* dyrow = dy + ((row0 + 16 * I + c) * H + h) * P;
#pragma unroll
          for (int kp = 0; kp < NKP; ++kp) frag_load_k<P>(fd[half][kp], dyrow, kp * 32 + 8 * q);
        }
      }
      Frag<T> fa;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int I = 2 * I2 + half;
        if (I >= J) {
          f4 dp = {0.f, 0.f, 0.f, 0.f}, dpt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kp = 0; kp < NKP; ++kp) {
            mma(dp, fd[half][kp], xf[kp]);   // lane: column j = cj, rows i = 16I + 4q + r
            mma(dpt, xf[kp], fd[half][kp]);  // lane: column i = 16I + c, rows j = rj0 + r
          }
          const int i0 = 16 * I + 4 * q;
          const f4 csi = *reinterpret_cast<const f4*>(&cs[i0]);
          const int ci = 16 * I + c;
          const float cs_ci = cs[ci];
          float rsum = 0.0f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float lam = (i0 + r >= cj) ? __expf(csi[r] - cs_cj) : 0.0f;
            const float pv = to_f(wv[half][r]) * lam;
            colsum += dp[r] * pv;
            frag_set<T>(fa, half * 4 + r, pv);
            const float lamt = (ci >= rj0 + r) ? __expf(cs_ci - cs_rj[r]) : 0.0f;
            rsum += dpt[r] * dt_rj[r] * (to_f(wtv[half][r]) * lamt);
          }
          rowpart[I] += rsum;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) frag_set<T>(fa, half * 4 + r, 0.0f);
        }
      }
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        Frag<T> fb;
        frag_load2(fb, &DYt[tp * 16 + c][32 * I2 + 4 * q], &DYt[tp * 16 + c][32 * I2 + 16 + 4 * q]);
        mma(adx[tp], fa, fb);
      }
    }
    colsum = sum_q(colsum) * dt_cj;
    if (q == 0) colacc[cj] = colsum;
    // ddt (direct part) and dx for rows j = 16J + 4q + r
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) {
      const int p = tp * 16 + c;
      const V4 xv = *reinterpret_cast<const V4*>(&Xt[p][16 * J + 4 * q]);
      const V4 dv = *reinterpret_cast<const V4*>(&DYt[p][16 * J + 4 * q]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * J + 4 * q + r;
        part[r] += adx[tp][r] * to_f(xv[r]);
        dx[((row0 + j) * H + h) * P + p] = from_f<T>(dts[j] * adx[tp][r] + Dh * to_f(dv[r]));
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float s = sum16(part[r]);
      if (c == 0) ddtd[16 * J + 4 * q + r] = s;
    }
  }
  // this wave's row sums: combine the 4 lane groups, add to the wave's row
#pragma unroll
  for (int I = 0; I < NT; ++I) {
    const float s = sum_q(rowpart[I]);
    if (q == 0) rowacc[wave][16 * I + c] += s;
  }

  // (3) <Gk, Hin_k> and sum <dy, x> over the chunk
  float gh = 0.0f, dd = 0.0f;
  for (int e = threadIdx.x; e < P * N; e += NTH) gh += to_f(Gs[e / N][e % N]) * to_f(Hs[e / N][e % N]);
  for (int e = threadIdx.x; e < P * Q; e += NTH) dd += to_f(DYt[e / Q][e % Q]) * to_f(Xt[e / Q][e % Q]);
  gh = wave_sum(gh);
  dd = wave_sum(dd);
  if (l == 0) { red[wave] = gh; red[NW + wave] = dd; }
  __syncthreads();

  // (4) assemble dcs, reverse cumsum, ddt, partial dA / dD (wave 0)
  if (wave == 0) {
    float ghs = 0.0f, dds = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) { ghs += red[w]; dds += red[NW + w]; }
    float qs = 0.0f;
#pragma unroll
    for (int t = 0; t < TPL; ++t) qs += qv[l * TPL + t];
    qs = wave_sum(qs);
    float v[TPL];
#pragma unroll
    for (int t = 0; t < TPL; ++t) {
      const int i = l * TPL + t;
      float rsum = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) rsum += rowacc[w][i];
      v[t] = rsum - colacc[i] - qv[i];
      if (i == Q - 1) v[t] += qs + __expf(cs_last) * ghs;
    }
    // local suffix sums, then across lanes
#pragma unroll
    for (int t = TPL - 2; t >= 0; --t) v[t] += v[t + 1];
    const float incl = wave_inclusive_suffix(v[0]);
    float excl = __shfl_down(incl, 1, kWave);
    if (l == kWave - 1) excl = 0.0f;
    const float Ah = Ap[h];
    float da = 0.0f;
#pragma unroll
    for (int t = 0; t < TPL; ++t) {
      const int j = l * TPL + t;
      const float dl = v[t] + excl;
      da += dts[j] * dl;
      ddt[(row0 + j) * H + h] = from_f<T>(Ah * dl + ddtd[j]);
    }
    da = wave_sum(da);
    if (l == 0) {
      dapart[bkh] = da;
      ddpart[bkh] = dds;
    }
  }
}

// ---------------------------------------------------------------------------
// Backward-order C.B^T tiles from the forward-order tiles the forward pass
// saved: a per-tile lane transpose through LDS, so both orders hold the same
// rounded values (tile (I, J): forward lane (q, c) holds W[16I + c][16J + 4q + r],
// backward lane (q, c) holds W[16I + 4q + r][16J + c]).
template <typename T, int Q>
__global__ __launch_bounds__(256) void k_tiles_to_bwd(const T* __restrict__ wf, T* __restrict__ wb, int nsplit) {
  constexpr int NT = Q / 16, TILES = NT * (NT + 1) / 2;
  __shared__ float tb[4][16][17];
  const int wave = threadIdx.x / kWave, l = lane_id(), q = l >> 4, c = l & 15;
  const int64_t base = (int64_t)blockIdx.x * TILES * 256;
  typedef typename Vec4<T>::type V4;
  for (int idx = blockIdx.y * 4 + wave; idx < TILES; idx += nsplit * 4) {
    const V4 v = *reinterpret_cast<const V4*>(wf + base + (int64_t)idx * 256 + l * 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) tb[wave][c][4 * q + r] = to_f(v[r]);  // tb[i_local][j_local]
    __builtin_amdgcn_wave_barrier();
    V4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = from_f<T>(tb[wave][4 * q + r][c]);
    *reinterpret_cast<V4*>(wb + base + (int64_t)idx * 256 + l * 4) = o;
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------------------
// Head-summed masked outer products for one (b, k, g) and one 64x64 block
// (IB, JB), JB <= IB, of the chunk's Q x Q matrix:
//   dW_ij = sum_{h in g} <dy_i, xt_j> exp(cs_i - cs_j)   (j <= i, else 0)
// Wave w owns the block's 16-row tile w; heads are the reduction loop.
template <typename T, int Q, int P>
__global__ __launch_bounds__(256) void k_dw(const T* __restrict__ x, const T* __restrict__ dt,
                                            const float* __restrict__ cs_g, const T* __restrict__ dy,
                                            float* __restrict__ dw, int L, int H, int G, int K) {
  constexpr int NKP = (P + 31) / 32;
  const int bkg = blockIdx.x;
  const int g = bkg % G, bk = bkg / G, k = bk % K, b = bk / K;
  int IB = 0;
  while ((IB + 1) * (IB + 2) / 2 <= (int)blockIdx.y) ++IB;
  const int JB = blockIdx.y - IB * (IB + 1) / 2;
  const int wave = threadIdx.x / kWave, l = lane_id(), q = l >> 4, c = l & 15;
  const int64_t row0 = (int64_t)b * L + (int64_t)k * Q;
  const int hpg = H / G;
  const int ib0 = 64 * IB + 16 * wave;  // first row of this wave's tile

  f4 acc[4];
#pragma unroll
  for (int tj = 0; tj < 4; ++tj) acc[tj] = f4{0.f, 0.f, 0.f, 0.f};

  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const float* csb = cs_g + (((int64_t)b * H + h) * K + k) * Q;
    Frag<T> fa[NKP];
    const T* dyrow = dy + ((row0 + ib0 + c) * H + h) * P;
#pragma unroll
    for (int kp = 0; kp < NKP; ++kp) frag_load_k<P>(fa[kp], dyrow, kp * 32 + 8 * q);
    const f4 csi = *reinterpret_cast<const f4*>(csb + ib0 + 4 * q);
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      if (IB == JB && tj > wave) continue;  // strictly above the diagonal: zero
      const int j = 64 * JB + 16 * tj + c;
      Frag<T> fb[NKP];
      const T* xrow = x + ((row0 + j) * H + h) * P;
#pragma unroll
      for (int kp = 0; kp < NKP; ++kp) frag_load_k<P>(fb[kp], xrow, kp * 32 + 8 * q);
      f4 dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kp = 0; kp < NKP; ++kp) mma(dp, fa[kp], fb[kp]);
      const float csj = csb[j];
      const float dtj = to_f(dt[(row0 + j) * H + h]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ib0 + 4 * q + r;
        const float lam = (i >= j) ? __expf(csi[r] - csj) : 0.0f;
        acc[tj][r] += dp[r] * dtj * lam;
      }
    }
  }
  float* o = dw + (int64_t)bkg * Q * Q;
#pragma unroll
  for (int tj = 0; tj < 4; ++tj) {
    const int j = 64 * JB + 16 * tj + c;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[(int64_t)(ib0 + 4 * q + r) * Q + j] = acc[tj][r];
  }
}

// ---------------------------------------------------------------------------
// dC / dB for one (b, k, g) and one 64-row block RB of the chunk:
//   dC_i = sum_{h in g} exp(cs_i) Hin_k^T dy_i + sum_{j <= i} dW_ij B_j
//   dB_j = sum_{h in g} e_j dt_j Gk^T x_j      + sum_{i >= j} dW_ij C_i
// The head sums are one product with K = (head, headdim): per head the rows
// (dy or x, pre-scaled) and the transposed state are staged in LDS.  Then the
// dW rows (or columns) and B (or C) are staged and multiplied with K = tokens.
template <typename T, int Q, int P, int N, bool DB>
__global__ __launch_bounds__(256) void k_dbc(const T* __restrict__ x, const T* __restrict__ dt,
                                             const float* __restrict__ cs_g, const T* __restrict__ dy,
                                             const T* __restrict__ state, const float* __restrict__ dw,
                                             const T* __restrict__ M, T* __restrict__ out,
                                             int L, int H, int G, int K) {
  constexpr int PAD = 16 / sizeof(T);
  constexpr int PP = P < 32 ? 32 : P;  // K extent of the head products, padded to a 32-step
  constexpr int TN = N / 16;
  constexpr size_t PH1 = sizeof(T) * (64 * (PP + PAD) + N * (PP + PAD));
  constexpr size_t PH2 = sizeof(T) * (64 * (Q + PAD) + N * (Q + PAD));
  constexpr size_t LDSB = PH1 > PH2 ? PH1 : PH2;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDSB];
  __shared__ float fac[64];
  T* As = reinterpret_cast<T*>(lds);                 // [64][PP + PAD]
  T* Ss = As + 64 * (PP + PAD);                      // [N][PP + PAD]
  T* Ws = reinterpret_cast<T*>(lds);                 // [64][Q + PAD]
  T* Mt = Ws + 64 * (Q + PAD);                       // [N][Q + PAD]

  const int bkg = blockIdx.x, RB = blockIdx.y;
  const int g = bkg % G, bk = bkg / G, k = bk % K, b = bk / K;
  const int wave = threadIdx.x / kWave, l = lane_id(), q = l >> 4, c = l & 15;
  const int64_t row0 = (int64_t)b * L + (int64_t)k * Q;
  const int r0 = 64 * RB;
  const int hpg = H / G;

  if (P < 32) {
    for (int e = threadIdx.x; e < (64 + N) * (PP + PAD); e += blockDim.x) As[e] = from_f<T>(0.0f);
  }
  f4 acc[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) acc[tn] = f4{0.f, 0.f, 0.f, 0.f};

  // phase 1: head sums (K = head x headdim)
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const float* csb = cs_g + (((int64_t)b * H + h) * K + k) * Q;
    __syncthreads();  // previous head's products are done with As / Ss / fac
    if (threadIdx.x < 64) {
      const int i = r0 + threadIdx.x;
      fac[threadIdx.x] = DB ? __expf(csb[Q - 1] - csb[i]) * to_f(dt[(row0 + i) * H + h]) : __expf(csb[i]);
    }
    __syncthreads();
    const T* rows = (DB ? x : dy) + ((row0 + r0) * H + h) * P;
    stage_rows<T, T, P, 256>(As, PP + PAD, rows, (int64_t)H * P, 64, fac);
    stage_transposed<T, T, N, 256>(Ss, PP + PAD, state + (((int64_t)b * K + k) * H + h) * P * N, N, P, nullptr);
    __syncthreads();
#pragma unroll
    for (int kp = 0; kp < PP / 32; ++kp) {
      Frag<T> fa;
      frag_load(fa, As + (16 * wave + c) * (PP + PAD) + kp * 32 + 8 * q);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        Frag<T> fb;
        frag_load(fb, Ss + (16 * tn + c) * (PP + PAD) + kp * 32 + 8 * q);
        mma(acc[tn], fa, fb);
      }
    }
  }
  __syncthreads();

  // phase 2: dW part (K = tokens)
  const float* dwb = dw + (int64_t)bkg * Q * Q;
  const int kb0 = DB ? r0 : 0;             // first token of the K range
  const int kr = DB ? Q - r0 : r0 + 64;    // K range length (multiple of 64)
  if (!DB) {
    // Ws[r][j] = dW[r0 + r][j];  Mt[n][j] = B[j][n]
    stage_rows<T, float, Q, 256>(Ws, Q + PAD, dwb + (int64_t)r0 * Q, Q, 64, nullptr);
  } else {
    // Ws[r][i - r0] = dW[i][r0 + r];  Mt[n][i - r0] = C[i][n]
    stage_transposed<T, float, 64, 256>(Ws, Q + PAD, dwb + (int64_t)r0 * Q + r0, Q, kr, nullptr);
  }
  stage_transposed<T, T, N, 256>(Mt, Q + PAD, M + ((row0 + kb0) * G + g) * N, (int64_t)G * N, kr, nullptr);
  __syncthreads();
  const int wofs = DB ? 0 : 0;
  for (int ks = 0; ks < kr / 32; ++ks) {
    Frag<T> fa;
    frag_load(fa, Ws + (16 * wave + c) * (Q + PAD) + wofs + ks * 32 + 8 * q);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      Frag<T> fb;
      frag_load(fb, Mt + (16 * tn + c) * (Q + PAD) + ks * 32 + 8 * q);
      mma(acc[tn], fa, fb);
    }
  }
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = r0 + 16 * wave + 4 * q + r;
      out[((row0 + row) * G + g) * N + 16 * tn + c] = from_f<T>(acc[tn][r]);
    }
  }
}

// Fixed-order sums of the per-(b, k) partials: one workgroup per head; each
// thread sums a strided slice, then a fixed tree combines the slices.
__global__ __launch_bounds__(256) void k_da_dd(const float* __restrict__ dapart, const float* __restrict__ ddpart,
                                               float* __restrict__ dA, float* __restrict__ dD, int BK, int H) {
  __shared__ float ra[4], rd[4];
  const int h = blockIdx.x;
  float sa = 0.0f, sd = 0.0f;
  for (int i = threadIdx.x; i < BK; i += 256) {
    sa += dapart[(int64_t)i * H + h];
    sd += ddpart[(int64_t)i * H + h];
  }
  sa = wave_sum(sa);
  sd = wave_sum(sd);
  const int wave = threadIdx.x / kWave;
  if (lane_id() == 0) { ra[wave] = sa; rd[wave] = sd; }
  __syncthreads();
  if (threadIdx.x == 0) {
    dA[h] = (ra[0] + ra[1]) + (ra[2] + ra[3]);
    dD[h] = (rd[0] + rd[1]) + (rd[2] + rd[3]);
  }
}

template <typename T, int Q, int P, int N>
void run_bwd(const Layout& lay, const BwdArgs& a, hipStream_t st, const ssd_probe* probe) {
  const int b = (int)lay.b, L = (int)lay.L, H = (int)lay.H, G = (int)lay.G, K = (int)lay.K;
  const T* x = static_cast<const T*>(a.x);
  const T* dt = static_cast<const T*>(a.dt);
  const T* B = static_cast<const T*>(a.B);
  const T* C = static_cast<const T*>(a.C);
  const T* dy = static_cast<const T*>(a.dy);
  const T* hin = static_cast<const T*>(a.hin);
  T* w = static_cast<T*>(a.w);
  T* gst = static_cast<T*>(a.gst);
  {
    ProbeScope ps(probe, SSD_K_BMM_BWD, st);
    const int nsplit = 4;
    k_tiles_to_bwd<T, Q><<<dim3(b * K * G, nsplit), dim3(256), 0, st>>>(static_cast<const T*>(a.wf), w, nsplit);
  }
  {
    ProbeScope ps(probe, SSD_K_CHUNK_STATE_BWD, st);
    k_chunk_state<T, Q, P, N, true><<<dim3(b * K * H), dim3(256), 0, st>>>(dy, C, dt, a.cs, a.dhloc, L, H, G, K);
  }
  {
    ProbeScope ps(probe, SSD_K_STATE_PASSING_BWD, st);
    const int PN = P * N;
    k_state_passing_bwd<T, Q><<<dim3((PN / 4 + 255) / 256, b * H), dim3(256), 0, st>>>(a.dhloc, a.cs, gst, H, K, PN);
  }
  {
    ProbeScope ps(probe, SSD_K_CHUNK_SCAN_BWD, st);
    k_chunk_scan_bwd<T, Q, P, N><<<dim3(b * K * H), dim3(256), 0, st>>>(
        x, dt, a.cs, a.A, a.D, B, C, hin, gst, static_cast<const T*>(a.wf), w, dy, static_cast<T*>(a.dx),
        static_cast<T*>(a.ddt),
        a.dapart, a.ddpart, L, H, G, K);
  }
  {
    ProbeScope ps(probe, SSD_K_DW, st);
    const int nb = Q / 64;
    k_dw<T, Q, P><<<dim3(b * K * G, nb * (nb + 1) / 2), dim3(256), 0, st>>>(x, dt, a.cs, dy, a.dw, L, H, G, K);
  }
  {
    ProbeScope ps(probe, SSD_K_DC, st);
    k_dbc<T, Q, P, N, false><<<dim3(b * K * G, Q / 64), dim3(256), 0, st>>>(
        x, dt, a.cs, dy, hin, a.dw, B, static_cast<T*>(a.dC), L, H, G, K);
  }
  {
    ProbeScope ps(probe, SSD_K_DB, st);
    k_dbc<T, Q, P, N, true><<<dim3(b * K * G, Q / 64), dim3(256), 0, st>>>(
        x, dt, a.cs, dy, gst, a.dw, C, static_cast<T*>(a.dB), L, H, G, K);
  }
  {
    ProbeScope ps(probe, SSD_K_DA_DD, st);
    k_da_dd<<<dim3(H), dim3(256), 0, st>>>(a.dapart, a.ddpart, a.dA, a.dD, b * K, H);
  }
}

#define SSD_INST_BWD_BF16(Q_, P_, N_) template void run_bwd<bf16, Q_, P_, N_>(const Layout&, const BwdArgs&, hipStream_t, const ssd_probe*);
#define SSD_INST_BWD_F32(Q_, P_, N_) template void run_bwd<float, Q_, P_, N_>(const Layout&, const BwdArgs&, hipStream_t, const ssd_probe*);
SSD_BF16_CONFIGS(SSD_INST_BWD_BF16)
SSD_F32_CONFIGS(SSD_INST_BWD_F32)

}  // namespace ssd
