// Kernels used by both the forward and the backward pass:
//   chunk cumsum, C.B^T tiles, chunk state (decay-weighted U^T V per chunk)
//   and the forward / reverse inter-chunk state scans.
#pragma once
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ssd {

template <typename T> __device__ __forceinline__ void frag_zero(Frag<T>& f);
template <> __device__ __forceinline__ void frag_zero<bf16>(Frag<bf16>& f) {
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = (bf16)0.0f;
}
template <> __device__ __forceinline__ void frag_zero<float>(Frag<float>& f) {
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = 0.0f;
}

// 8 contiguous K-values starting at k0 of a row whose K-extent is KD; zero
// beyond KD (KD = 16 leaves the upper half of a 32-wide step empty).
template <int KD, typename T, typename TI>
__device__ __forceinline__ void frag_load_k(Frag<T>& f, const TI* row, int k0) {
  if (KD % 32 == 0 || k0 < KD) frag_load(f, row + k0);
  else frag_zero(f);
}

// Chained-mapping fragment of a row (K-values k0 + 4q + s for s < 4 and
// k0 + 16 + 4q + s - 4 for s >= 4); with KD = 16 the second run is zero.
template <int KD, typename T>
__device__ __forceinline__ void frag_load_chained(Frag<T>& f, const T* row, int k0, int q) {
  if constexpr (KD % 32 == 0) {
    frag_load2(f, row + k0 + 4 * q, row + k0 + 16 + 4 * q);
  } else {
    static_assert(KD == 16, "K extent must be 16 or a multiple of 32");
    const typename Vec4<T>::type a = *reinterpret_cast<const typename Vec4<T>::type*>(row + k0 + 4 * q);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      frag_set<T>(f, s, to_f(a[s]));
      frag_set<T>(f, s + 4, 0.0f);
    }
  }
}

// The same from eight OCP E4M3 codes (two runs of four bytes), widened to bf16
// exactly (gfx950's packed conversion at scale 1).
template <int KD>
__device__ __forceinline__ void frag_load_chained(Frag<bf16>& f, const fp8* row, int k0, int q) {
  const uint32_t a = *reinterpret_cast<const uint32_t*>(row + k0 + 4 * q);
  uint32_t b = 0;  // E4M3 code 0 is +0
  if constexpr (KD % 32 == 0) b = *reinterpret_cast<const uint32_t*>(row + k0 + 16 + 4 * q);
  else static_assert(KD == 16, "K extent must be 16 or a multiple of 32");
  f.v = e4m3x8_to_bf16(make_uint2(a, b));
}

// First row of chunk k of sequence b, and the tensor that holds it: the
// caller's for whole chunks, the zero-padded copy for a shorter last chunk.
__device__ __forceinline__ int64_t chunk_row0(const RowMap& rm, int b, int k, int Q) {
  return k == rm.kf ? (int64_t)b * Q : (int64_t)b * rm.L + (int64_t)k * Q;
}
template <typename T>
__device__ __forceinline__ const T* rows_in(const RowMap& rm, int k, const T* p, const void* tail) {
  return k == rm.kf ? static_cast<const T*>(tail) : p;
}
template <typename T>
__device__ __forceinline__ T* rows_out(const RowMap& rm, int k, T* p, void* tail) {
  return k == rm.kf ? static_cast<T*>(tail) : p;
}

// Index of the lower-triangle 16x16 tile (I, J), J <= I.
__device__ __forceinline__ int tri_index(int I, int J) { return I * (I + 1) / 2 + J; }

// ---------------------------------------------------------------------------
// Chunk cumsum: cs[b][h][k][i] = sum_{j <= i} dt[b][kQ + j][h] * A[h].
// One wavefront per (b, HW adjacent heads, k); each lane owns Q/64
// consecutive tokens (one HW-wide load per token: the heads' steps of a token
// are adjacent in the caller's token-major dt) and the chunk-wide prefix of
// each head comes from a wave64 shuffle scan.
// The step is written in float32 for every later kernel, in cs's layout
// (dt_out[b][h][k][i], so that a chunk's steps of one head are contiguous;
// rows past the end of a shorter last chunk get 0).  It is the caller's dt
// widened or, with softplus set (dt then holds the raw step),
// softplus(dt + dt_bias[h]) = log(1 + e^z) (z itself above 20).
template <typename T, int Q, int HW>
__device__ __forceinline__ void chunk_cumsum_wave(const T* __restrict__ dt, const float* __restrict__ A,
                                                  const float* __restrict__ dt_bias, float* __restrict__ dt_out,
                                                  float* __restrict__ cs, const RowMap& rm, int H, int K, int softplus,
                                                  int item) {
  constexpr int TPL = Q / kWave;
  static_assert(HW == 1 || HW == 4, "heads per wave");
  const int HQ = H / HW;
  const int k = item % K, bq = item / K, h0 = (bq % HQ) * HW, b = bq / HQ;
  const int l = lane_id();
  const bool last = k == rm.kf;
  const int64_t row0 = chunk_row0(rm, b, k, Q);
  const T* src = rows_in(rm, k, dt, rm.dt);
  float a[HW], bias[HW];
#pragma unroll
  for (int w = 0; w < HW; ++w) {
    a[w] = A[h0 + w];
    bias[w] = (softplus && dt_bias) ? dt_bias[h0 + w] : 0.0f;
  }
  float v[HW][TPL];
#pragma unroll
  for (int j = 0; j < TPL; ++j) {
    const int i = l * TPL + j;
    const int64_t e = (row0 + i) * H + h0;
    float d[HW];
    if constexpr (HW == 4) {
      const typename Vec4<T>::type d4 = *reinterpret_cast<const typename Vec4<T>::type*>(src + e);
#pragma unroll
      for (int w = 0; w < HW; ++w) d[w] = to_f(d4[w]);
    } else {
      d[0] = to_f(src[e]);
    }
#pragma unroll
    for (int w = 0; w < HW; ++w) {
      if (softplus) {
        const float z = d[w] + bias[w];
        d[w] = z > 20.0f ? z : log1pf(expf(z));
      }
      if (last && i >= rm.lr) d[w] = 0.0f;
      v[w][j] = d[w];
    }
  }
#pragma unroll
  for (int w = 0; w < HW; ++w) {
    const int64_t bhk = ((int64_t)b * H + h0 + w) * K + k;
    float* dst = dt_out + bhk * Q + l * TPL;
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
      dst[j] = v[w][j];
      v[w][j] *= a[w];
    }
#pragma unroll
    for (int j = 1; j < TPL; ++j) v[w][j] += v[w][j - 1];
    const float incl = wave_inclusive_scan(v[w][TPL - 1]);
    float excl = __shfl_up(incl, 1, kWave);
    if (l == 0) excl = 0.0f;
    float* out = cs + bhk * Q + l * TPL;
#pragma unroll
    for (int j = 0; j < TPL; ++j) out[j] = v[w][j] + excl;
  }
}

// Rows staged in LDS as 16-byte pieces (NPC pieces per row of N elements of
// type TI, CRPP rows per 256 bytes of LDS): piece p of row r is stored at
// p ^ row_swz(r), so that the 16 rows of one fragment read (lane (q, c) reads
// row c) meet distinct banks.
template <int NPC, int CRPP>
__device__ __forceinline__ int row_swz(int r) {
  if constexpr (NPC == 1) return 0;
  else return (r / CRPP) & ((NPC < 16 ? NPC : 16) - 1);
}
// Element offset of K-value kk of staged row r.
template <int N, int NPC, int CRPP, typename TI>
__device__ __forceinline__ int staged_off(int r, int kk) {
  constexpr int EP = 16 / sizeof(TI);
  return r * N + ((kk / EP) ^ row_swz<NPC, CRPP>(r)) * EP + kk % EP;
}
// Fragment of staged row r with K-values k0 .. k0 + 7 (zero past N): one
// piece for bf16 and FP8 (widened), two for fp32.
template <int N, int NPC, int CRPP, typename T, typename TI>
__device__ __forceinline__ void staged_row_frag(Frag<T>& f, const TI* rows, int r, int k0) {
  if (N % 32 == 0 || k0 < N) {
    if constexpr (sizeof(TI) == 4) frag_load2(f, rows + staged_off<N, NPC, CRPP, TI>(r, k0), rows + staged_off<N, NPC, CRPP, TI>(r, k0 + 4));
    else frag_load(f, rows + staged_off<N, NPC, CRPP, TI>(r, k0));
  } else {
    frag_zero(f);
  }
}

// ---------------------------------------------------------------------------
// W = C.B^T per (b, k, g), stored as lower-triangle 16x16 accumulator tiles in
// the lane order the forward chunk kernel reads (4 elements per lane, 256 per
// tile): tile (I, J) lane l holds W[16I + l%16][16J + 4q + r] (q = l / 16,
// r = 0..3), K = dstate.  Only k_chunk_scan_fwd reads these: the chunk scan
// resident over heads forms the same tiles itself, and the backward forms
// its tiles again in fp32 from C and B.
// One workgroup per (b, k, g) and four consecutive row tiles I = 4m + wave:
// each wave holds the C fragments of its row tile in registers, and the B rows
// stream through LDS in 64-row blocks (blocks 0 .. m), so every B and C row
// is fetched once per workgroup instead of once per tile.  With FP8 (E4M3) B
// and C the products run on the FP8 matrix cores, whose fragment is the bf16
// one with one byte per K-value (checked on gfx950: OCP E4M3 operands, lane
// (q, c) supplies row c, K-values 8q .. 8q + 7).
template <typename TI, int N>
struct BmmLds {
  __attribute__((aligned(16))) TI Bs[64 * N];
};

template <typename T, typename TI, int Q, int N>
__device__ __forceinline__ void bmm_rows_block(const TI* __restrict__ B, const TI* __restrict__ C, T* __restrict__ wf,
                                               const RowMap& rm, int G, int K, int bkg, int m, BmmLds<TI, N>& sm) {
  constexpr int NTH = 256;
  constexpr int NT = Q / 16, TILES = NT * (NT + 1) / 2;
  constexpr int NK = (N + 31) / 32;
  constexpr bool F8 = std::is_same<TI, fp8>::value;
  constexpr int EP = 16 / sizeof(TI);
  constexpr int RBY = N * (int)sizeof(TI);
  constexpr int NPC = RBY / 16, CRPP = RBY >= 256 ? 1 : 256 / RBY;
  constexpr int PIECES = 64 * NPC, PPT = (PIECES + NTH - 1) / NTH;
  static_assert(RBY % 16 == 0, "B rows are whole 16-byte pieces");
  const int g = bkg % G, bk = bkg / G, k = bk % K, b = bk / K;
  const int wave = threadIdx.x / kWave, l = lane_id(), q = l >> 4, c = l & 15;
  const int I = 4 * m + wave;
  const int64_t row0 = chunk_row0(rm, b, k, Q);
  B = rows_in(rm, k, B, rm.B);
  C = rows_in(rm, k, C, rm.C);
  const TI* crow = C + ((row0 + 16 * I + c) * G + g) * N;
  // C fragments of row tile I (the product's second operand: column c = row 16 I + c)
  [[maybe_unused]] long c8[F8 ? NK : 1];
  [[maybe_unused]] Frag<T> cf[F8 ? 1 : NK];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    const int kk = ks * 32 + 8 * q;
    if constexpr (F8) c8[ks] = (N % 32 == 0 || kk < N) ? *reinterpret_cast<const long*>(crow + kk) : 0;
    else frag_load_k<N>(cf[ks], crow, kk);
  }
  T* out = wf + (int64_t)bkg * TILES * 256 + l * 4;
  for (int jb = 0; jb <= m; ++jb) {
    if (jb > 0) __syncthreads();  // the previous block's rows are no longer read
#pragma unroll
    for (int n = 0; n < PPT; ++n) {
      const int u = threadIdx.x + NTH * n;
      if (PIECES % NTH == 0 || u < PIECES) {
        const int r = u / NPC;
        *reinterpret_cast<uint4*>(&sm.Bs[u * EP]) = *reinterpret_cast<const uint4*>(
            B + ((row0 + 64 * jb + r) * G + g) * N + ((u % NPC) ^ row_swz<NPC, CRPP>(r)) * EP);
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int J = 4 * jb + t;
      if (J > I) break;  // wave-uniform
      f4 af = {0.f, 0.f, 0.f, 0.f};
      const int r = 16 * t + c;  // B row 16 J + c of the staged block
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const int kk = ks * 32 + 8 * q;
        if constexpr (F8) {
          const long b8 = (N % 32 == 0 || kk < N) ? *reinterpret_cast<const long*>(&sm.Bs[staged_off<N, NPC, CRPP, TI>(r, kk)]) : 0;
          af = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(b8, c8[ks], af, 0, 0, 0);
        } else {
          Frag<T> fb;
          staged_row_frag<N, NPC, CRPP>(fb, &sm.Bs[0], r, kk);
          mma(af, fb, cf[ks]);  // [row j][col i] = B_j . C_i
        }
      }
      typename Vec4<T>::type v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = from_f<T>(af[e]);
      *reinterpret_cast<typename Vec4<T>::type*>(out + (int64_t)tri_index(I, J) * 256) = v;
    }
  }
}

// The two independent first steps of the forward in one launch:
// workgroups [0, nbmm) compute C.B^T tiles (workgroup = (b, k, g) and four
// consecutive row tiles), the rest the chunk cumsum, one wave per (b, HW
// heads, k).  Both are small and latency-bound, so their waves overlap
// instead of running as two launches one after the other.  The Q/64 C.B^T
// workgroups of one (b, k, g), which stage the same B rows, are dealt 8
// dispatch slots apart (one XCD and its L2, about the same time; the
// heaviest first), nbmm = Q/64 times the item count rounded up to 8.
template <typename T, typename TI, int Q, int N, int HW>
__global__ __launch_bounds__(256) void k_cumsum_bmm(const T* __restrict__ dt, const float* __restrict__ A,
                                                    const float* __restrict__ dt_bias, float* __restrict__ dt_out,
                                                    float* __restrict__ cs, const TI* __restrict__ B,
                                                    const TI* __restrict__ C, T* __restrict__ wf,
                                                    const RowMap rm, int H, int G, int K, int softplus, int nbkg,
                                                    int nbhk) {
  constexpr int NM = Q / 64;  // groups of four row tiles
  static_assert(Q % 64 == 0, "chunk");
  __shared__ BmmLds<TI, N> sm;
  const int nbmm = (nbkg + 7) / 8 * 8 * NM;
  if ((int)blockIdx.x < nbmm) {
    const int xcd = blockIdx.x % 8, j = blockIdx.x / 8;
    const int item = (j / NM) * 8 + xcd;
    if (item >= nbkg) return;  // whole workgroup, before any barrier
    bmm_rows_block<T, TI, Q, N>(B, C, wf, rm, G, K, item, NM - 1 - j % NM, sm);
  } else {
    const int item = ((int)blockIdx.x - nbmm) * 4 + threadIdx.x / kWave;
    if (item < nbhk / HW) chunk_cumsum_wave<T, Q, HW>(dt, A, dt_bias, dt_out, cs, rm, H, K, softplus, item);
  }
}

// ---------------------------------------------------------------------------
// Chunk state: out[b][k][h][p][n] = sum_i w_i U[kQ+i][h][p] V[kQ+i][g][n]
//   forward  (BWD = false): U = x,  V = B, w_i = dt_i exp(cs_{Q-1} - cs_i)
//   backward (BWD = true) : U = dy, V = C, w_i = exp(cs_i)
// The backward also forms, from the same staged rows, each token's
// state-to-output term of the chunk-scan gradient
//   t_i = exp(cs_i) <dy_i, Hin_k^T C_i>      (Hin_k: the chunk's entry state)
// as (Hin C^T) tiles with K = dstate, one headdim tile per wave: wave w
// writes its 16 headdim columns' share of t_i, and the chunk-scan gradient's
// dl assembly adds the shares.
// A (P x Q)(Q x N) product on the matrix cores with K = tokens.  Both
// operands have K as their outer index in memory, so KB-token blocks of U
// (rows scaled by w_i on the way) and V are staged row-major in LDS and both
// fragments are read K-major with the transposing LDS read.  Blocks are
// double-buffered: the next block is loaded into registers while the
// current one is used.  One workgroup (4 waves) per (b, k) and HPW heads of
// one group: V, the group's rows, is staged once for all of them, and their U
// rows are one contiguous run per token.
template <typename T, typename TU, typename TV, int Q, int P, int N, bool BWD, int HPW>
__global__ __launch_bounds__(256) void k_chunk_state(const TU* __restrict__ U, const TV* __restrict__ V,
                                                     const float* __restrict__ dt, const float* __restrict__ cs,
                                                     T* __restrict__ out, const T* __restrict__ hin,
                                                     float* __restrict__ dlpart, const RowMap rm, int H, int G, int K,
                                                     int nitems) {
  constexpr int NTH = 256;
  // tokens per block: the forward's smaller blocks at dstate 128 fit more
  // workgroups on a CU (long context 0.268 -> 0.258 ms); the backward, which
  // also forms the state-to-output rows per block, measured slower with them
  // (0.38 -> 0.40 ms), and so did the forward at dstate 64
  constexpr int KB = (!BWD && N >= 128) ? 32 : 64;
  constexpr int NB = Q / KB;
  constexpr int UP = P + 16, VP = N + 16;          // row pitches (8 mod 16 dwords for 64 / 128 wide rows)
  constexpr int TM = P / 16, TN = N / 16, NT = TM * TN, TPW = (NT + 3) / 4;
  constexpr int VN = Vec16<T>::n;
  constexpr int UPIECES = KB * P / VN, VPIECES = KB * N / VN;
  constexpr int UPT = (UPIECES + NTH - 1) / NTH, VPT = (VPIECES + NTH - 1) / NTH;
  typedef typename Vec16<T>::type V16;
  __shared__ __attribute__((aligned(16))) T Us[2][HPW][KB][UP];
  __shared__ __attribute__((aligned(16))) T Vs[2][KB][VP];
  // backward: the state-to-output term's headdim-tile shares of a block,
  // summed over the tiles after the next barrier and written as one row
  constexpr int TPHS = BWD ? P / 16 : 1;
  __shared__ float TS[BWD ? 2 : 1][BWD ? HPW : 1][TPHS][BWD ? KB : 1];

  const int bkhp = xcd_item(blockIdx.x, nitems);
  if (bkhp >= nitems) return;  // whole workgroup, before any barrier
  const int HP = H / HPW;
  const int hp = bkhp % HP, bk = bkhp / HP, k = bk % K, b = bk / K;
  const int h0 = hp * HPW;                         // HPW consecutive heads, one group
  const int g = h0 / (H / G);
  const int wave = threadIdx.x / kWave, l = lane_id(), q = l >> 4, c = l & 15;
  const int64_t row0 = chunk_row0(rm, b, k, Q);
  U = rows_in(rm, k, U, BWD ? rm.dy : rm.x);
  V = rows_in(rm, k, V, BWD ? rm.C : rm.B);
  const float* csc[HPW];
  const float* dtc[HPW];
  float cs_last[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    csc[hh] = cs + (((int64_t)b * H + h0 + hh) * K + k) * Q;
    dtc[hh] = dt + (((int64_t)b * H + h0 + hh) * K + k) * Q;
    cs_last[hh] = csc[hh][Q - 1];
  }

  // backward: Hin rows 16 w .. 16 w + 15 of each head as A fragments (K = dstate)
  constexpr int NKN = (N + 31) / 32, TPH = P / 16;
  [[maybe_unused]] Frag<T> hfr[BWD ? HPW : 1][BWD ? NKN : 1];
  if constexpr (BWD) {
    if (wave < TPH) {
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
        for (int ks = 0; ks < NKN; ++ks)
          frag_load_k<N>(hfr[hh][ks], hin + ((((int64_t)b * K + k) * H + h0 + hh) * P + 16 * wave + c) * N, ks * 32 + 8 * q);
    }
  }

  V16 uv[HPW][UPT], vv[VPT];
  float uw[HPW][UPT];
  auto load = [&](int blk) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
      for (int n = 0; n < UPT; ++n) {
        const int u = threadIdx.x + NTH * n;
        if (UPIECES % NTH == 0 || u < UPIECES) {
          const int i = KB * blk + u / (P / VN);
          uv[hh][n] = load_vec16<T, TU>(U + ((row0 + i) * H + h0 + hh) * P + (u % (P / VN)) * VN);
          uw[hh][n] = BWD ? __expf(csc[hh][i]) : dtc[hh][i] * __expf(cs_last[hh] - csc[hh][i]);
        }
      }
    }
#pragma unroll
    for (int n = 0; n < VPT; ++n) {
      const int u = threadIdx.x + NTH * n;
      if (VPIECES % NTH == 0 || u < VPIECES)
        vv[n] = load_vec16<T, TV>(V + ((row0 + KB * blk + u / (N / VN)) * G + g) * N + (u % (N / VN)) * VN);
    }
  };
  auto store = [&](int bf) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
      for (int n = 0; n < UPT; ++n) {
        const int u = threadIdx.x + NTH * n;
        if (UPIECES % NTH == 0 || u < UPIECES) {
          V16 w;
#pragma unroll
          for (int e = 0; e < VN; ++e) w[e] = from_f<T>(to_f(uv[hh][n][e]) * uw[hh][n]);
          *reinterpret_cast<V16*>(&Us[bf][hh][u / (P / VN)][(u % (P / VN)) * VN]) = w;
        }
      }
    }
#pragma unroll
    for (int n = 0; n < VPT; ++n) {
      const int u = threadIdx.x + NTH * n;
      if (VPIECES % NTH == 0 || u < VPIECES)
        *reinterpret_cast<V16*>(&Vs[bf][u / (N / VN)][(u % (N / VN)) * VN]) = vv[n];
    }
  };

  f4 acc[HPW][TPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[hh][t] = f4{0.f, 0.f, 0.f, 0.f};

  // the shares of block sblk (in TS[sblk & 1]) summed over the headdim tiles
  // in tile order and written (after a barrier that follows their writes)
  auto ts_write = [&](int sblk) {
    if constexpr (BWD) {
      constexpr int NSP = scan_bwd_splits(Q);
      const int hh = threadIdx.x / KB, i = threadIdx.x % KB;
      if (hh < HPW) {
        float v = TS[sblk & 1][hh][0][i];
#pragma unroll
        for (int w = 1; w < TPHS; ++w) v += TS[sblk & 1][hh][w][i];
        const int64_t bkhh = ((int64_t)b * K + k) * H + h0 + hh;
        dlpart[(bkhh * dl_rows(Q) + NSP + 3) * Q + KB * sblk + i] = v;
      }
    }
  };
  load(0);
  store(0);
  for (int blk = 0; blk < NB; ++blk) {
    const int bf = blk & 1;
    __syncthreads();  // block blk is in buffer bf; buffer bf ^ 1 is no longer read
    if (blk > 0) ts_write(blk - 1);
    if (blk + 1 < NB) load(blk + 1);
#pragma unroll
    for (int ks = 0; ks < KB / 32; ++ks) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int j = wave + 4 * t;
        if (j < NT) {
          const int tm = j / TN, tn = j % TN;
          Frag<T> fb;
          frag_load_kmajor<32>(fb, &Vs[bf][0][0], VP, ks * 32, tn * 16, q, c);
#pragma unroll
          for (int hh = 0; hh < HPW; ++hh) {
            Frag<T> fa;
            frag_load_kmajor<32>(fa, &Us[bf][hh][0][0], UP, ks * 32, tm * 16, q, c);
            mma(acc[hh][t], fa, fb);
          }
        }
      }
    }
    if constexpr (BWD) {
      // state-to-output term of the block's tokens, headdim tile `wave`:
      // m[r] = (Hin C^T)[p = 16 wave + 4q + r][i = 16 rt + c], times the staged
      // exp(cs_i) dy_i[p] and summed over p; the tile's share goes to TS
      static_assert(TPH == TPHS && HPW * KB <= NTH, "shares summed by one thread per token and head");
      if (wave < TPH) {
#pragma unroll
        for (int rt = 0; rt < KB / 16; ++rt) {
          Frag<T> fc[NKN];
#pragma unroll
          for (int ks = 0; ks < NKN; ++ks) frag_load_k<N>(fc[ks], &Vs[bf][16 * rt + c][0], ks * 32 + 8 * q);
#pragma unroll
          for (int hh = 0; hh < HPW; ++hh) {
            f4 m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKN; ++ks) mma(m, hfr[hh][ks], fc[ks]);
            const typename Vec4<T>::type u = *reinterpret_cast<const typename Vec4<T>::type*>(&Us[bf][hh][16 * rt + c][16 * wave + 4 * q]);
            float t = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) t += m[r] * to_f(u[r]);
            t = sum_q(t);
            if (q == 0) TS[bf][hh][wave][16 * rt + c] = t;
          }
        }
      }
    }
    if (blk + 1 < NB) store(bf ^ 1);
  }
  if constexpr (BWD) {
    __syncthreads();
    ts_write(NB - 1);
  }
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    T* o = out + (((int64_t)b * K + k) * H + h0 + hh) * P * N;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int j = wave + 4 * t;
      if (j < NT) {
        const int tm = j / TN, tn = j % TN;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[(tm * 16 + 4 * q + r) * N + tn * 16 + c] = from_f<T>(acc[hh][t][r]);
      }
    }
  }
}

// Head slices of a kernel resident over heads: about one workgroup per CU
// where the (b, k, g) items are few, one slice per item where they are many,
// at most 64 heads a slice.  Returns the heads per slice; *S the slice count.
// Such a kernel pays when a slice holds at least kMinResidentHeads heads to
// spread its group operands' staging over (measured on the forward chunk
// scan: 20, 14 and 10 heads faster than one workgroup per head, 8 slower).
constexpr int kMinResidentHeads = 10;
// The chunk-scan backward resident over heads pays from fewer heads: 8 (the
// Mamba2-370M shape) measured 0.154 -> 0.122 ms; fewer were not measured.
constexpr int kMinResidentHeadsBwd = 8;
inline int resident_slices(int nbkg, int hpg, int* S) {
  int s = (256 + nbkg - 1) / nbkg;
  if (s > hpg) s = hpg;
  int per = (hpg + s - 1) / s;
  if (per > 64) per = 64;
  *S = (hpg + per - 1) / per;
  return per;
}

// Launch of k_chunk_state: two heads per workgroup when a group's heads pair up.
// hin / dlpart: the backward's chunk-entry states and dl partial sums (the
// state-to-output term), unused (null) in the forward.
template <typename T, typename TU, typename TV, int Q, int P, int N, bool BWD>
void launch_chunk_state(const TU* U, const TV* V, const float* dt, const float* cs, T* out, const T* hin,
                        float* dlpart, const RowMap& rm, int b, int H, int G, int K, hipStream_t st) {
  if ((H / G) % 2 == 0)
    k_chunk_state<T, TU, TV, Q, P, N, BWD, 2><<<dim3(xcd_grid(b * K * H / 2)), dim3(256), 0, st>>>(
        U, V, dt, cs, out, hin, dlpart, rm, H, G, K, b * K * H / 2);
  else
    k_chunk_state<T, TU, TV, Q, P, N, BWD, 1><<<dim3(xcd_grid(b * K * H)), dim3(256), 0, st>>>(
        U, V, dt, cs, out, hin, dlpart, rm, H, G, K, b * K * H);
}

// ---------------------------------------------------------------------------
// Inter-chunk state passing, elementwise over the P*N state entries of each
// (b, h) and sequential over chunks.
//   forward:        h = init (zero if null); for k = 0 .. K-1:
//                     out[k] = h;  h = exp(cs_{Q-1}(k)) h + in[k];      final = h
//                   (in = the chunk states S, out = Hin)
//   reverse (BWD):  g = dfinal (zero if null); for k = K-1 .. 0:
//                     out[k] = g;  g = in[k] + exp(cs_{Q-1}(k)) g;      final = g
//                   (in = dH_loc, out = G, the gradient w.r.t. the state
//                   leaving chunk k; the final g is the initial-state gradient)
// Each thread owns 4 consecutive entries; inputs and outputs are in the
// storage type, the carry is float32.
// The chain through the chunks is sequential, and a launch has only
// b * H * P * N / 4 threads (2560 waves at 80 heads of 64 x 128 states), so a
// wave that waited for each chunk's load before the next would leave HBM
// mostly idle.  Loads run kScanAhead chunks ahead of the one being added,
// through a ring of registers (the loop is unrolled by the ring length so
// every slot is a fixed register set).  The log-decays of a block of
// kScanAhead chunks arrive as one vector load, lane l holding chunk l of the
// block, and are read with readlane: as scalar loads (which may return out
// of order) every use would wait for all of them.
constexpr int kScanAhead = 16;

template <typename T, int Q, bool BWD>
__global__ __launch_bounds__(256) void k_state_passing(const T* __restrict__ in, const float* __restrict__ cs,
                                                       const float* __restrict__ init, T* __restrict__ out,
                                                       float* __restrict__ fin, int H, int K, int PN) {
  typedef typename Vec4<T>::type V;
  constexpr int D = kScanAhead;
  const int e = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (e >= PN) return;
  const int bh = blockIdx.y, h = bh % H, b = bh / H, l = lane_id();
  const float* csb = cs + (int64_t)bh * K * Q + (Q - 1);
  const int64_t stride = (int64_t)H * PN;  // one chunk further
  const T* src = in + ((int64_t)b * K * H + h) * PN + e;
  T* dst = out + ((int64_t)b * K * H + h) * PN + e;
  auto chunk = [&](int i) { return BWD ? K - 1 - i : i; };  // chunk of step i
  // log-decay of step i0 + l % D (clamped to the last step), lane l
  auto lg_load = [&](int i0) { return csb[(int64_t)chunk(min(i0 + l % D, K - 1)) * Q]; };
  f4 st = {0.f, 0.f, 0.f, 0.f};
  if (init) st = *reinterpret_cast<const f4*>(init + (int64_t)bh * PN + e);
  // the slot is consumed before its refill is issued, so the refill can land
  // in the same registers (no copy, which would wait for the load)
  auto step = [&](V& slot, int i, float lgv, int u, bool refill) {
    const float alpha = __expf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(lgv), u)));
    V v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = from_f<T>(st[r]);
    *reinterpret_cast<V*>(dst + chunk(i) * stride) = v;
#pragma unroll
    for (int r = 0; r < 4; ++r) st[r] = alpha * st[r] + to_f(slot[r]);
    if (refill) slot = *reinterpret_cast<const V*>(src + chunk(i + D) * stride);
  };
  V ring[D];
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (u < K) ring[u] = *reinterpret_cast<const V*>(src + chunk(u) * stride);
  float lgv = lg_load(0);
  int i0 = 0;
  // every refill of these blocks is in range
  for (; i0 + 2 * D <= K; i0 += D) {
    const float lgn = lg_load(i0 + D);
#pragma unroll
    for (int u = 0; u < D; ++u) step(ring[u], i0 + u, lgv, u, true);
    lgv = lgn;
  }
  for (; i0 < K; i0 += D) {
    const float lgn = i0 + D < K ? lg_load(i0 + D) : 0.0f;
#pragma unroll
    for (int u = 0; u < D; ++u)
      if (i0 + u < K) step(ring[u], i0 + u, lgv, u, i0 + u + D < K);
    lgv = lgn;
  }
  if (fin) *reinterpret_cast<f4*>(fin + (int64_t)bh * PN + e) = st;
}

}  // namespace ssd
