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

// ---------------------------------------------------------------------------
// The same chunk scan for bf16 with headdim 64, resident over heads: one
// workgroup of 8 waves (one per CU, 2 waves per SIMD) per (b, k, g) and
// slice of the group's heads.  Each wave keeps the C fragments and the C.B^T
// tiles of its two row tiles in registers for the whole slice (the group's
// operands, read once per slice instead of once per head), and the heads
// stream through two LDS buffers: each head's x rows, entering state and step
// / cumsum values are copied from global memory straight into LDS (no
// registers) one head ahead, while the current head's products run.  Per
// head a workgroup then reads only that head's rows, about 50 KB instead of
// the 200 KB a per-head workgroup requests.  The products are those of
// k_chunk_scan_fwd.  With one wave per SIMD (4 waves) the products' LDS and
// exponential latencies stayed exposed (0.20 against 0.16 ms at the 2.7B
// shape); with 8 waves the copy addresses are formed from 32-bit per-thread
// offsets so the kernel stays within 256 registers without spilling.
template <int Q, int N>
struct FwdGroupLayout {
  static constexpr int P = 64;
  static constexpr int XPIECES = Q * P / 8, HPIECES = P * N / 8;  // 16-byte pieces (bf16)
  static constexpr int NW = 8, NTH = NW * 64;                     // 8 waves: 2 per SIMD
  static constexpr int XPT = XPIECES / NTH, HPT = HPIECES / NTH;   // copies per thread and head
  static constexpr int X8T = Q * P / 16 / NTH;                    // FP8 x: 16-code loads per thread
  static_assert(XPIECES % NTH == 0 && HPIECES % NTH == 0 && (Q * P / 16) % NTH == 0, "whole copies per thread");
};

// x in bf16 (TI = bf16) is copied into LDS directly; FP8 x, B and C (TI =
// fp8): x is loaded into registers with the next head's copies, widened to
// bf16 and stored into the other buffer after the current head's products,
// and the resident C fragments are widened as they are loaded.
template <typename TI, int Q, int N>
__global__ __launch_bounds__(512, 1) void k_chunk_scan_fwd_heads(
    const TI* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ cs_g,
    const float* __restrict__ Dp, const TI* __restrict__ C, const TI* __restrict__ B, const bf16* __restrict__ hin,
    bf16* __restrict__ y, const RowMap rm, int H, int G, int K, int hps, int nslice, int nbkg) {
  typedef bf16 T;
  typedef FwdGroupLayout<Q, N> Ly;
  constexpr int P = Ly::P;
  constexpr int NTH = Ly::NTH, NW = Ly::NW;
  constexpr int NT = Q / 16, TP = P / 16;
  constexpr int NK = N / 32, NJ2 = NT / 2;
  constexpr int NSLOT = NT / NW;  // row tiles per wave
  constexpr int XPT = Ly::XPT, HPT = Ly::HPT, X8T = Ly::X8T;
  constexpr bool F8 = std::is_same<TI, fp8>::value;
  constexpr int HPC = N / 8;      // 16-byte pieces of a state row
  constexpr int YST = NSLOT * TP;  // y stores of one head per thread (8-byte, never merged)
  static_assert(N % 32 == 0 && NT % NW == 0 && YST < 64, "shape");
  typedef typename Vec4<T>::type V4;
  // Two head buffers, each one object (see the head loop).
  struct alignas(16) Buf {
    T X[Q * P];             // x rows, xcol-permuted
    T H[P * N];             // Hin, pieces XOR-permuted by row
    float S[2 * Q + 4 * kWave];  // cs [0, Q), dt [Q, 2Q); the other waves' copies land past them, unread
    float F[Q];                  // bfac
  };
  __shared__ Buf B0, B1;
  __shared__ float Ds[64];  // D of the slice's heads

  const int xcd = blockIdx.x % 8, jb = blockIdx.x / 8;
  const int slice = jb % nslice, bkg = (jb / nslice) * 8 + xcd;
  if (bkg >= nbkg) return;  // whole workgroup, before any barrier
  const int g = bkg % G, bk = bkg / G, k = bk % K, b = bk / K;
  const int hpg = H / G, h0 = g * hpg + slice * hps, nh = min(hps, hpg - slice * hps);
  const int wave = threadIdx.x / kWave, l = lane_id(), q = l >> 4, c = l & 15;
  const int64_t row0 = chunk_row0(rm, b, k, Q);
  x = rows_in(rm, k, x, rm.x);
  C = rows_in(rm, k, C, rm.C);
  B = rows_in(rm, k, B, rm.B);
  y = rows_out(rm, k, y, rm.y);

  int Is[NSLOT];
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) Is[sl] = 2 * NW * (sl / 2) + ((sl & 1) ? 2 * NW - 1 - wave : wave);

  // ---- the group's operands of this wave's row tiles, resident: the C
  // fragments, and the tiles W = C.B^T of its row tiles, formed here from
  // the chunk's B rows staged in the two x buffers (the products, their
  // order and the rounding to bf16 of the C.B^T tile kernel)
  constexpr int RBY = N * (int)sizeof(TI), NPC = RBY / 16, EPC = 16 / (int)sizeof(TI);
  constexpr int XBP = Q * P * 2 / 16, BPT = Q * NPC / NTH;  // 16-byte pieces of an x buffer; B copies per thread
  static_assert(Q * RBY <= 2 * Q * P * 2 && XBP % NTH == 0 && BPT * NTH == Q * NPC && (NTH / NPC) % NPC == 0,
                "B rows fit the two x buffers");
  Frag<T> cf[NSLOT][NK];
  V4 wv[NSLOT][NT];
  // slot sl's row tile never exceeds jm(sl) - 1 (zig-zag), so only its tiles
  // J < jm(sl) are held (the rest are never referenced and take no registers)
  auto jm = [&](int sl) { return 2 * NW * (sl / 2) + ((sl & 1) ? 2 * NW : NW); };
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) {
    const TI* crow = C + ((row0 + 16 * Is[sl] + c) * G + g) * N;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) frag_load_k<N>(cf[sl][ks], crow, ks * 32 + 8 * q);
  }
  {
    // B row j, piece pl at LDS piece pl ^ (j mod NPC): rows of the first
    // XBP pieces in B0.X, the rest in B1.X
    const int t = threadIdx.x, bj0 = t / NPC, bo0 = bj0 * G * N + ((t % NPC) ^ (bj0 & (NPC - 1))) * EPC;
    const TI* bg = B + (row0 * G + g) * N;
#pragma unroll
    for (int n = 0; n < BPT; ++n) {
      const int u0 = n * NTH;
      unsigned char* dst = (u0 < XBP ? reinterpret_cast<unsigned char*>(B0.X) : reinterpret_cast<unsigned char*>(B1.X)) +
                           ((u0 % XBP) + wave * kWave) * 16;
      lds_copy16(bg + bo0 + (int64_t)(u0 / NPC) * G * N, dst);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0070);
  __syncthreads();
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) {
    const int I = Is[sl];
#pragma unroll
    for (int J = 0; J < NT; ++J) {
      if (J >= jm(sl)) continue;
      f4 af = {0.f, 0.f, 0.f, 0.f};
      if (J <= I) {  // tiles past the diagonal are never used
        const int r = 16 * J + c, u = r * NPC;
        const unsigned char* rowp = (u < XBP ? reinterpret_cast<const unsigned char*>(B0.X)
                                             : reinterpret_cast<const unsigned char*>(B1.X)) + (u % XBP) * 16;
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          Frag<T> fb;
          if constexpr (F8) {
            const int pc = (2 * ks + (q >> 1)) ^ (r & (NPC - 1));
            fb.v = e4m3x8_to_bf16(*reinterpret_cast<const uint2*>(rowp + pc * 16 + 8 * (q & 1)));
          } else {
            fb.v = *reinterpret_cast<const bf16x8*>(rowp + (((4 * ks + q) ^ (r & (NPC - 1))) * 16));
          }
          mma(af, fb, cf[sl][ks]);  // [row j][col i] = B_j . C_i
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) wv[sl][J][e] = from_f<T>(af[e]);
    }
  }
  __syncthreads();  // the B rows are no longer read: the x buffers take the heads
  if (threadIdx.x < nh) Ds[threadIdx.x] = Dp[h0 + threadIdx.x];

  // ---- one head's copies into a buffer: thread t's 16 bytes of copy n land
  // at byte 16 (n NTH + t) of the array, so it fetches the piece the permuted
  // layout keeps there.  Copy n of a thread reads 64 n / (P / 8) rows (x) or
  // NTH / (N / 8) n rows (Hin) below copy 0, and the row permutations depend
  // only on row bits the step does not change, so each source is a 32-bit
  // per-thread offset plus a multiple of a uniform stride.  Every thread
  // issues DPH copies per head.
  static_assert(NTH % (P / 8) == 0 && NTH % HPC == 0 && (NTH / (P / 8)) % 16 == 0 && (NTH / HPC) % HPC == 0,
                "copy steps keep the permutation bits");
  const int t = threadIdx.x;
  const int xr0 = t / (P / 8), xo0 = xr0 * H * P + ((t % (P / 8)) ^ (2 * ((xr0 ^ (xr0 >> 2)) & 3))) * 8;
  const int xstep = (NTH / (P / 8)) * H * P;
  const int hr0 = t / HPC, ho0 = hr0 * N + ((t % HPC) ^ (hr0 & (HPC - 1))) * 8;
  // cs then dt (2 Q floats) from the first Q / 128 waves; every other wave
  // issues the same copy (so all waves count the same copies per head) into
  // the spare tail of the buffer's S, which nothing reads
  const int su = t < Q / 2 ? t : 0;
  static_assert(Q / 2 % kWave == 0, "whole waves copy cs and dt");
  auto head_dma = [&](int hh, T* Xb, T* Hb, float* Sb) {
    const int h = h0 + hh;
    if constexpr (!F8) {
      const TI* xh = x + (row0 * H + h) * P;
#pragma unroll
      for (int n = 0; n < XPT; ++n) lds_copy16(xh + xo0 + n * xstep, Xb + (n * NTH + wave * kWave) * 8);
    }
    const T* hs = hin + ((((int64_t)b * K + k) * H + h) * P) * N;
#pragma unroll
    for (int n = 0; n < HPT; ++n) lds_copy16(hs + ho0 + n * (NTH / HPC) * N, Hb + (n * NTH + wave * kWave) * 8);
    const float* csb = cs_g + (((int64_t)b * H + h) * K + k) * Q;
    const float* dtb = dt + (((int64_t)b * H + h) * K + k) * Q;
    lds_copy16(su < Q / 4 ? csb + 4 * su : dtb + 4 * (su - Q / 4), Sb + min(wave, Q / 128) * kWave * 4);
  };
  // FP8 x: 16 codes (a quarter row) per load, widened into the xcol-permuted rows
  [[maybe_unused]] uint4 x8[F8 ? X8T : 1];
  auto x8_load = [&](int hh) {
    const int h = h0 + hh;
#pragma unroll
    for (int n = 0; n < X8T; ++n) {
      const int u = t + NTH * n, r = u / (P / 16), cq = (u % (P / 16)) * 16;
      x8[n] = *reinterpret_cast<const uint4*>(x + ((row0 + r) * H + h) * P + cq);
    }
  };
  auto x8_store = [&](T* Xb) {
#pragma unroll
    for (int n = 0; n < X8T; ++n) {
      const int u = t + NTH * n, r = u / (P / 16), cq = (u % (P / 16)) * 16;
      *reinterpret_cast<bf16x8*>(&Xb[r * P + xcol(r, cq)]) = e4m3x8_to_bf16(make_uint2(x8[n].x, x8[n].y));
      *reinterpret_cast<bf16x8*>(&Xb[r * P + xcol(r, cq + 8)]) = e4m3x8_to_bf16(make_uint2(x8[n].z, x8[n].w));
    }
  };

  int xoff[TP];
#pragma unroll
  for (int tp = 0; tp < TP; ++tp) {
    const int r0 = 4 * q + (c >> 2);
    xoff[tp] = r0 * P + xcol(r0, 16 * tp + 4 * (c & 3));
  }

  // one head from the buffer (Xb, Hb, Sb, Fb)
  auto head = [&](int hh, const T* Xb, const T* Hb, const float* Sb, float* Fb) {
    const int h = h0 + hh;
    const float* csl = Sb;
    const float* dtl = Sb + Q;
    // bfac_j = dt_j exp(cs_r - cs_j), r the last token of j's 32-token step
#pragma unroll
    for (int i = threadIdx.x; i < Q; i += NTH) Fb[i] = __expf(csl[i | 31] - csl[i]) * dtl[i];
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const float Dh = Ds[hh];
    T* yh = y + h * P;
    // The per-lane values pass through an empty asm at every head, so the
    // addresses formed from them are formed here instead of being hoisted
    // out of the head loop, one set per buffer (hoisted, they spilled, and
    // the spill reloads in the loop waited for every copy)
    int c = lane_id() & 15, q = lane_id() >> 4, xo[TP];
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) xo[tp] = xoff[tp];
    asm volatile("" : "+v"(c), "+v"(q));
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) asm volatile("" : "+v"(xo[tp]));
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) {
      const int I = Is[sl];
      f4 acc[TP];
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) acc[tp] = f4{0.f, 0.f, 0.f, 0.f};
      // 1. state -> output: Hin . C_i (K = dstate); lane column i = 16I + c
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
#pragma unroll
        for (int tp = 0; tp < TP; ++tp) {
          const int r = 16 * tp + c;
          Frag<T> fh;
          frag_load(fh, Hb + r * N + ((4 * ks + q) ^ (r & (HPC - 1))) * 8);
          mma(acc[tp], fh, cf[sl][ks]);
        }
      }
      const int ci = 16 * I + c;
      const float cs_i = csl[ci];
      {
        const float e = __expf(cs_i);
#pragma unroll
        for (int tp = 0; tp < TP; ++tp) acc[tp] *= e;
      }
      // 2. intra-chunk, steps of 32 source tokens (as in k_chunk_scan_fwd)
#pragma unroll
      for (int J2 = 0; J2 < NJ2; ++J2) {
        if (2 * J2 >= jm(sl) || 2 * J2 > I) break;
        Frag<T> fa;
        if (2 * J2 + 1 < I) {
          const float ai = __expf(cs_i - csl[32 * J2 + 31]);
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int J = 2 * J2 + half;
            const f4 bj = *reinterpret_cast<const f4*>(&Fb[16 * J + 4 * q]);
#pragma unroll
            for (int r = 0; r < 4; ++r) frag_set<T>(fa, half * 4 + r, to_f(wv[sl][J][r]) * (ai * bj[r]));
          }
        } else {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int J = 2 * J2 + half;
            const int j0 = 16 * J + 4 * q;
            const f4 csj = *reinterpret_cast<const f4*>(&csl[j0]);
            const f4 dtj = *reinterpret_cast<const f4*>(&dtl[j0]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float m = (J <= I && j0 + r <= ci) ? __expf(cs_i - csj[r]) * dtj[r] : 0.0f;
              frag_set<T>(fa, half * 4 + r, to_f(wv[sl][J][r]) * m);
            }
          }
        }
#pragma unroll
        for (int tp = 0; tp < TP; ++tp) {
          Frag<T> fx;
          const T* a = Xb + 32 * J2 * P + xo[tp];
          frag_load_kmajor_at(fx, a, a + 16 * P);
          mma(acc[tp], fx, fa);
        }
      }
      // 3. + D x, store y[i][16tp + 4q + r]
      T* yr = yh + (row0 + ci) * H * P;
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        const V4 xv = *reinterpret_cast<const V4*>(&Xb[ci * P + xcol(ci, 16 * tp + 4 * q)]);
        V4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = from_f<T>(acc[tp][r] + Dh * to_f(xv[r]));
        *reinterpret_cast<V4*>(yr + 16 * tp + 4 * q) = o;
      }
    }
  };

  // ---- heads.  Head hh lives in buffer hh & 1.  At the top of a head, its
  // copies have landed once at most the previous head's y stores (issued
  // after them) are in flight; after the barrier the other buffer is free
  // (the previous head is done with it) and takes the next head's copies.
  // The loop is unrolled by two so that every LDS access names its buffer,
  // and the compiler does not wait for copies into the other one.  (Three
  // buffers, the copies two heads ahead, measured slower: 0.128 -> 0.138 ms
  // at the 2.7B shape.)
  head_dma(0, B0.X, B0.H, B0.S);
  if constexpr (F8) {
    x8_load(0);
    x8_store(B0.X);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): resident operands and head 0
  __syncthreads();                     // Ds, head 0's copies
  auto step = [&](int hh, Buf& Bc, Buf& Bn) {
    if (hh > 0) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(YST));
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    if (hh + 1 < nh) {
      head_dma(hh + 1, Bn.X, Bn.H, Bn.S);
      if constexpr (F8) x8_load(hh + 1);
    }
    head(hh, Bc.X, Bc.H, Bc.S, Bc.F);
    // FP8: head hh + 1's x rows into the other buffer, free since the
    // barrier above; the next barrier publishes them.  Their loads, issued
    // after head hh + 1's copies, are waited for here, and with them those
    // copies (vmcnt counts in order), so the next wait stays correct.
    if constexpr (F8) {
      if (hh + 1 < nh) x8_store(Bn.X);
    }
  };
  for (int hh = 0; hh < nh; hh += 2) {
    step(hh, B0, B1);
    if (hh + 1 < nh) step(hh + 1, B1, B0);
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
  // The chunk scan resident over heads where a slice holds enough heads
  // (resident_slices): measured 20 heads (2.7B shape) 0.156 -> 0.130 ms, 14
  // (Zamba2-7B-like) 89 -> 82 us, 10 (long context) 0.583 -> 0.529 ms, but 8
  // (Mamba2-370M shape) 57 -> 59 us.  It forms its C.B^T tiles itself, so
  // the first launch then computes the cumsum only.
  int S = 1;
  const int per = resident_slices(b * K * G, H / G, &S);
  const bool resident = std::is_same<T, bf16>::value && P == 64 && N % 32 == 0 && per >= kMinResidentHeads;
  {
    ProbeScope ps(probe, SSD_K_CUMSUM_BMM, st);
    const int nbkg = resident ? 0 : b * K * G, nbhk = b * H * K, nbmm = (nbkg + 7) / 8 * 8 * (Q / 64);
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
    const int nbkg = b * K * G;
    if (resident) {
      if constexpr (std::is_same<T, bf16>::value && P == 64 && N % 32 == 0)
        k_chunk_scan_fwd_heads<TI, Q, N><<<dim3((nbkg + 7) / 8 * 8 * S), dim3(FwdGroupLayout<Q, N>::NTH), 0, st>>>(
            x, dt, a.cs, a.D, C, B, hin, static_cast<T*>(a.y), a.rows, H, G, K, per, S, nbkg);
    } else {
      k_chunk_scan_fwd<T, TI, Q, P, N><<<dim3(xcd_grid(b * K * H)), dim3(256), 0, st>>>(
          x, dt, a.cs, a.D, C, hin, wt, static_cast<T*>(a.y), a.rows, H, G, K, b * K * H);
    }
  }
}

#define SSD_INST_FWD_BF16(Q_, P_, N_) template void run_fwd<bf16, bf16, Q_, P_, N_>(const Layout&, const FwdArgs&, hipStream_t, const ssd_probe*);
#define SSD_INST_FWD_FP8(Q_, P_, N_) template void run_fwd<bf16, fp8, Q_, P_, N_>(const Layout&, const FwdArgs&, hipStream_t, const ssd_probe*);
#define SSD_INST_FWD_F32(Q_, P_, N_) template void run_fwd<float, float, Q_, P_, N_>(const Layout&, const FwdArgs&, hipStream_t, const ssd_probe*);
SSD_BF16_CONFIGS(SSD_INST_FWD_BF16)
SSD_BF16_CONFIGS(SSD_INST_FWD_FP8)
SSD_F32_CONFIGS(SSD_INST_FWD_F32)

}  // namespace ssd
