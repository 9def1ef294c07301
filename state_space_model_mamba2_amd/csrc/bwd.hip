// Backward pass of the SSD chunked scan.
#include "kern_shared.h"

namespace ssd {

// ---------------------------------------------------------------------------
// Per-head chunk backward.  With Gk = dL/d(state leaving chunk k),
// xt_j = dt_j x_j, W_ij = C_i . B_j, Lam_ij = exp(cs_i - cs_j) (j <= i) and
// P = W o Lam:
//   dxt_j = e_j B_j^T Gk + sum_{i >= j} P_ij dy_i,        e_j = exp(cs_{Q-1} - cs_j)
//   R_ij  = <dy_i, xt_j> P_ij
//   dcs_i = sum_j R_ij - sum_i' R_i'i + exp(cs_i) <dy_i, Hin_k^T C_i> - q_i,
//           q_j = <xt_j, e_j B_j^T Gk>;   dcs_{Q-1} += sum_j q_j + exp(cs_{Q-1}) <Gk, Hin_k>
//   dl    = reverse cumsum of dcs inside the chunk
//   ddt_j = A dl_j + <dxt_j, x_j>,  dx_j = dt_j dxt_j + D dy_j
// This kernel writes dx and, per token, the partial sums that dl is formed
// from (row sums, column sums, q_j, <dxt_j, x_j>); the state-to-output term
// exp(cs_i) <dy_i, Hin^T C_i> comes from the chunk-state gradient kernel,
// which has dy and C staged already, and k_dl_assemble finishes dl, ddt and
// the chunk's dA / dD partials.
//
// Layout of the work.  NSPLIT workgroups of 4 waves share one (b, k, h);
// the chunk's 16-token column tiles J are dealt to the 4 NSPLIT waves in a
// zig-zag (owner o gets J = o and 2 NO - 1 - o), so the triangular work is
// even.  A wave keeps, per owned tile, x_J as fragments and dxt_J^T as
// matrix-core accumulators whose rows are the same headdim entries (lane
// (q, c) holds dxt[16J + c][16tp + 4q + r], or with bf16 and headdim 64 the
// permuted rows 32 (tp / 2) + 8q + 4 (tp % 2) + r, which makes x one 16-byte
// load), so every token's x and dxt values sit in the same lane and slot:
// <dxt_j, x_j> and q_j need no second read of x.
// This head's dy rows and the group's C rows stream through LDS in 32-row
// slabs from the chunk end backwards (C mostly hits in L2, which it shares
// with the other heads of the group).  W is formed per tile pair on the
// matrix cores in fp32 from those C rows and the owned B_J fragments, which
// stay in registers from the state term: dA sums R over the whole chunk with
// much cancellation between row sums, column sums and the state terms, and
// C.B^T rounded to bf16 moved dA by up to 3 % of its largest head.  bf16 with headdim 64 copies the
// slabs from global memory straight into LDS (global_load_lds, 16 bytes per
// lane written at the wave's LDS base + 16 * lane: no registers, no LDS
// stores) three slabs ahead of the one in use, into four buffers; every
// other shape stages one slab ahead through registers.  The loop keeps its
// global stores (dx and the per-token sums) until after its last slab, so
// the only memory operations in flight in it are these copies and a slab is
// known to have landed once at most the copies issued after it are
// outstanding.  Every use of dy falls in the
// slab being processed, so LDS holds two slabs of it, not the whole chunk;
// the dy^T operands come from it through transposing reads.  A column tile's dxt is complete once the slab holding its
// own rows has been used, so dx is written right there.
// R is formed once per (I, J) tile pair on the matrix cores: lanes own a
// column j, so column sums accumulate in-lane and row sums come from 16-lane
// register (DPP) reductions over the very same values; the diagonal R_jj
// (which cancels exactly between the two) is left out of both.
// The workgroups of one (b, k, h) are 8 dispatch slots apart, so the
// round-robin dispatch over the 8 XCDs runs them on one XCD (one L2) at
// about the same time, and consecutive heads of a chunk (which share its C
// and B rows and C.B^T tiles) run on the same XCD.
template <typename T, typename TI, int Q, int P, int N>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void k_chunk_scan_bwd(
    const TI* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ cs_g, const float* __restrict__ Dp,
    const TI* __restrict__ B, const TI* __restrict__ C, const T* __restrict__ hin, const T* __restrict__ gst,
    const T* __restrict__ dy, T* __restrict__ dx, float* __restrict__ dlpart,
    float* __restrict__ dlscal, int nitems, const RowMap rm, int H, int G, int K) {
  constexpr int NW = 4, NTH = NW * kWave;
  constexpr int NSPLIT = scan_bwd_splits(Q);
  constexpr int PADR = 16 / sizeof(T);    // row padding: 16-byte aligned rows, spread banks
  constexpr int NT = Q / 16, NS = NT / 2, TP = P / 16, TILES = NT * (NT + 1) / 2;
  constexpr int NK = (N + 31) / 32, NKP = (P + 31) / 32;
  constexpr int NO = NSPLIT * NW;         // column-tile owners per (b, k, h)
  constexpr int NSLOT = NT / NO;          // column tiles per wave
  constexpr int SR = 32;                  // rows per slab
  constexpr int VN = Vec16<T>::n;
  constexpr int CUP = P / VN;
  constexpr int YPIECES = SR * CUP;       // 16-byte pieces of a dy slab
  // dy rows.  bf16 with headdim 64: unpadded, the 16-byte pieces of row r
  // XOR-permuted by f(r) = 2 ((r / 2) mod 4) + (r / 8) mod 2, so that the
  // transposing dy^T reads (per half-wave 8 rows x 32 bytes) and the row
  // fragment reads (16 rows x 16 bytes) both meet every bank once.  Otherwise a
  // pitch of 8 (mod 16) dwords, which serves the transposing reads.
  constexpr bool DSWZ = sizeof(T) == 2 && P == 64;
  constexpr int DPITCH = DSWZ ? P : sizeof(T) == 2 ? P + 2 * ((24 - (P / 2) % 16) % 16) : P + PADR;
  constexpr bool DMA = DSWZ;               // slabs copied global -> LDS directly
  // XC (bf16, headdim 64): the rows of dxt^T tile tp are permuted so that lane
  // (q, c) holds headdim entries 32 (tp / 2) + 8 q + 4 (tp % 2) + r, r < 4: the
  // two tiles of a 32-wide K step give each lane 8 consecutive entries, so
  // x is one 16-byte load per fragment (instead of two 8-byte pieces), a dy
  // row fragment one 16-byte LDS read and dx one 16-byte store.  Row m of
  // tile tp is headdim entry xrow(tp, m).
  constexpr bool XC = DSWZ;
  auto xrow = [](int tp, int m) { return 32 * (tp >> 1) + 8 * (m >> 2) + 4 * (tp & 1) + (m & 3); };
  constexpr int PF = DMA ? 3 : 1;          // slabs in flight ahead of the one in use
  constexpr int NBUF = DMA ? PF + 1 : 2;   // slab buffers
  constexpr int YPT = (YPIECES + NTH - 1) / NTH;
  // C rows of a slab, in their storage type: 16-byte pieces of EP elements,
  // NPC per row, piece p of row r stored at p ^ row_swz(r) so that the 16 rows
  // of a fragment read meet distinct banks.  The last round of copies fills
  // a spare tail of the buffer when a slab has fewer pieces than threads.
  constexpr int EP = 16 / sizeof(TI);
  constexpr int RBY = N * (int)sizeof(TI);  // bytes per C row
  constexpr int NPC = RBY / 16;
  constexpr int CRPP = RBY >= 256 ? 1 : 256 / RBY;  // C rows per 256 bytes
  constexpr int CPIECES = SR * NPC;
  constexpr int CPT = (CPIECES + NTH - 1) / NTH;
  constexpr int CSLAB = CPT * NTH * EP;
  static_assert(RBY % 16 == 0, "C rows are whole 16-byte pieces");
  static_assert(P == 16 || P % 32 == 0, "headdim");
  static_assert(N == 16 || N % 32 == 0, "dstate");
  static_assert(NT % NO == 0 && NSLOT >= 1 && NS >= 1, "chunk");
  static_assert(NSLOT == 1 || NSLOT == 2, "zig-zag dealing of two tiles per owner");
  static_assert(TP <= NW, "each Hin row block needs a wave");
  static_assert(NSPLIT == 1 || NSPLIT == 2, "a split owns one row tile of each slab");
  typedef typename Vec4<T>::type V4;
  typedef typename Vec16<T>::type V;
  typedef uint4 CV;  // a 16-byte piece of C
  // slab buffers: this head's dy rows and the group's C rows of the slab.
  // Each buffer is an array of its own, and the slab loop is unrolled over
  // them, so the compiler can tell the buffer being read from the ones being
  // filled by copies in flight (it does not wait for a copy before an LDS
  // read of another array)
  __shared__ __attribute__((aligned(16))) T DY0[SR][DPITCH], DY1[SR][DPITCH];
  __shared__ __attribute__((aligned(16))) T DY2[DMA ? SR : 1][DPITCH], DY3[DMA ? SR : 1][DPITCH];
  __shared__ __attribute__((aligned(16))) TI W0[CSLAB], W1[CSLAB];
  __shared__ __attribute__((aligned(16))) TI W2[DMA ? CSLAB : 1], W3[DMA ? CSLAB : 1];
  // Gk (DMA path): read by every wave, so it is copied into LDS once instead
  // of each wave fetching all of it; 16-byte pieces of row r XOR-permuted by
  // r mod (N / 8), so the 16 rows of a fragment read meet distinct banks
  __shared__ __attribute__((aligned(16))) T GS[DMA ? P : 1][DMA ? N : 1];
  static_assert(NBUF == 2 || NBUF == 4, "slab buffers");
  __shared__ __attribute__((aligned(16))) float cs[Q];
  __shared__ __attribute__((aligned(16))) float dts[Q];
  __shared__ __attribute__((aligned(16))) float ecs[Q];    // exp(cs_i)
  __shared__ __attribute__((aligned(16))) float eslab[Q];  // exp(cs_i - cs_rb), rb = first row of i's slab
  __shared__ float rowacc[NW][Q];
  __shared__ float red[2 * NW];
  // storage column of dy element (r, col) of a slab
  auto dyc = [](int r, int col) { return DSWZ ? col ^ (8 * ((((r >> 1) & 3) << 1) | ((r >> 3) & 1))) : col; };

  // (b, k, h) item and column split of this workgroup: the XCD-aware item
  // map (consecutive heads of a chunk on one XCD) over groups of NSPLIT * 8
  // workgroups, in which the splits of an item are 8 slots apart (one XCD)
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int split = slot % NSPLIT;
  const int bkh = xcd_item(kXcds * (slot / NSPLIT) + xcd, nitems);
  if (bkh >= nitems) return;  // whole workgroup, before any barrier
  const int h = bkh % H, bk = bkh / H, k = bk % K, b = bk / K;
  const int g = h / (H / G);
  const int wave = threadIdx.x / kWave, l = lane_id(), q = l >> 4, c = l & 15;
  const int64_t row0 = chunk_row0(rm, b, k, Q);
  x = rows_in(rm, k, x, rm.x);
  const float* dtc = dt + (((int64_t)b * H + h) * K + k) * Q;
  B = rows_in(rm, k, B, rm.B);
  C = rows_in(rm, k, C, rm.C);
  dy = rows_in(rm, k, dy, rm.dy);
  dx = rows_out(rm, k, dx, rm.dx);
  const int64_t rs = (int64_t)H * P;      // row stride of x / dy / dx
  const T* dyh = dy + (row0 * H + h) * P;  // row i of this chunk and head: dyh + i * rs
  const TI* xh = x + (row0 * H + h) * P;
  const TI* cg = C + row0 * G * N + g * N;  // C row i of this chunk and group: cg + i * G * N
  const T* hinh = hin + (int64_t)bkh * P * N;
  const T* gsth = gst + (int64_t)bkh * P * N;
  float* part = dlpart + (int64_t)bkh * dl_rows(Q) * Q;  // rows: splits' row sums, column sums, q, <dxt, x>

  // column tile of wave w, slot sl, in this split
  auto tile_of = [&](int w, int sl) {
    const int o = split * NW + w;
    return (sl & 1) ? 2 * NO - 1 - o : o;
  };
  int Js[NSLOT];
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) Js[sl] = tile_of(wave, sl);

  // ---- slab staging: registers <- global (a slab ahead of the one next in
  // LDS), LDS <- registers
  // global piece held at position u (< CPIECES) of a C slab buffer: row u / NPC
  auto c_src = [&](int s, int u) {
    const int r = u / NPC;
    return cg + (int64_t)(SR * s + r) * G * N + ((u % NPC) ^ row_swz<NPC, CRPP>(r)) * EP;
  };
  struct SlabRegs { V yv[YPT]; CV cv[CPT]; };
  SlabRegs ra;
  auto slab_load = [&](SlabRegs& R, int s) {
#pragma unroll
    for (int n = 0; n < YPT; ++n) {
      const int u = threadIdx.x + NTH * n;
      if (YPIECES % NTH == 0 || u < YPIECES)
        R.yv[n] = *reinterpret_cast<const V*>(dyh + (int64_t)(SR * s + u / CUP) * rs + (u % CUP) * VN);
    }
#pragma unroll
    for (int n = 0; n < CPT; ++n) {
      const int u = threadIdx.x + NTH * n;
      if (CPIECES % NTH == 0 || u < CPIECES) R.cv[n] = *reinterpret_cast<const CV*>(c_src(s, u));
    }
  };
  auto slab_store = [&](const SlabRegs& R, T (*dyb)[DPITCH], TI* cb) {
#pragma unroll
    for (int n = 0; n < YPT; ++n) {
      const int u = threadIdx.x + NTH * n;
      if (YPIECES % NTH == 0 || u < YPIECES)
        *reinterpret_cast<V*>(&dyb[u / CUP][dyc(u / CUP, (u % CUP) * VN)]) = R.yv[n];
    }
#pragma unroll
    for (int n = 0; n < CPT; ++n) {
      const int u = threadIdx.x + NTH * n;
      if (CPIECES % NTH == 0 || u < CPIECES) *reinterpret_cast<CV*>(&cb[u * EP]) = R.cv[n];
    }
  };
  // global -> LDS copies of slab s into buffer (dyb, cb): thread t's 16 bytes land at
  // byte 16 t of the buffer, so it fetches the piece the swizzled layout keeps
  // there (dy row t / 8, LDS piece t % 8 holds global piece (t % 8) ^ f(row);
  // C alike with row_swz).  Every thread issues the same number of copies, so one
  // vmcnt threshold fits every wave: positions past the slab's pieces fetch
  // a copy of an earlier piece into the buffer's spare tail.
  constexpr int DPS = YPT + CPT;           // copies per thread and slab
  static_assert(!DMA || (YPIECES == NTH && 2 * DPS <= 15), "slab copies");
  auto slab_dma = [&](int s, T (*dyb)[DPITCH], TI* cb) {
    const int t = threadIdx.x, r = t / CUP;
    const int kp = (t % CUP) ^ ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
    lds_copy16(dyh + (int64_t)(SR * s + r) * rs + kp * VN, &dyb[0][0] + wave * kWave * VN);
#pragma unroll
    for (int n = 0; n < CPT; ++n) {
      const int u = t + NTH * n;
      lds_copy16(c_src(s, u % CPIECES), &cb[(NTH * n + wave * kWave) * EP]);
    }
  };

  // ---- prologue.  Every global load of the prologue is issued first, in one
  // straight-line block, so they are all in flight together; LDS stores and
  // products follow.
  constexpr int QPT = (Q + NTH - 1) / NTH;
  const float* csc = cs_g + (((int64_t)b * H + h) * K + k) * Q;
  float csv[QPT], dtv[QPT];
#pragma unroll
  for (int n = 0; n < QPT; ++n) {
    const int i = threadIdx.x + NTH * n;
    if (Q % NTH == 0 || i < Q) {
      csv[n] = csc[i];
      dtv[n] = dtc[i];
    }
  }
  constexpr int GPC = N / VN;  // 16-byte pieces of a G row
  if constexpr (DMA) {
    static_assert((P * GPC) % NTH == 0 && (GPC & (GPC - 1)) == 0, "G copy");
#pragma unroll
    for (int n = 0; n < P * GPC / NTH; ++n) {
      const int pp = n * NTH + threadIdx.x, r = pp / GPC, pc = (pp % GPC) ^ (r & (GPC - 1));
      lds_copy16(gsth + r * N + pc * VN, &GS[0][0] + (n * NTH + wave * kWave) * VN);
    }
  } else {
    slab_load(ra, NS - 1);
  }
  Frag<T> xf[NSLOT][NKP];
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl)
#pragma unroll
    for (int kp = 0; kp < NKP; ++kp) {
      if constexpr (XC) frag_load(xf[sl][kp], xh + (int64_t)(16 * Js[sl] + c) * rs + kp * 32 + 8 * q);
      else frag_load_chained<P>(xf[sl][kp], xh + (int64_t)(16 * Js[sl] + c) * rs, kp * 32, q);
    }
  // Hin rows 16 w .. 16 w + 15 (split 0, waves 0 .. TP-1: their share of <Gk, Hin>)
  const bool gh_wave = split == 0 && wave < TP;
  Frag<T> hf[NK];
  if (gh_wave) {
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      frag_load_k<N>(hf[ks], hinh + (XC ? xrow(wave, c) : 16 * wave + c) * N, ks * 32 + 8 * q);
  }
  [[maybe_unused]] Frag<T> gf[DMA ? 1 : NK][TP];
  Frag<T> bfr[NK][NSLOT];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    if constexpr (!DMA) {
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) frag_load_k<N>(gf[ks][tp], gsth + (16 * tp + c) * N, ks * 32 + 8 * q);
    }
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl)
      frag_load_k<N>(bfr[ks][sl], B + ((row0 + 16 * Js[sl] + c) * G + g) * N, ks * 32 + 8 * q);
  }
  // fragment of Gk rows 16 tp .. 16 tp + 15, K-values ks * 32 + 8q .. (lane (q, c))
  auto gfrag = [&](Frag<T>& f, int ks, int tp) {
    if constexpr (DMA) {
      const int r = XC ? xrow(tp, c) : 16 * tp + c;
      frag_load(f, &GS[r][(((ks * 32 + 8 * q) / VN) ^ (r & (GPC - 1))) * VN]);
    } else {
      f = gf[ks][tp];
    }
  };

  // LDS stores of the per-token scalars (their loads were issued first) and
  // the row factors every slab uses, formed once here instead of by every
  // lane of a 16-lane group in every slab
  static_assert(SR == 32 && kWave % SR == 0 && NTH % SR == 0, "a slab's first row sits in the same wave");
#pragma unroll
  for (int n = 0; n < QPT; ++n) {
    const int i = threadIdx.x + NTH * n;
    const float csr = __shfl(csv[n], l & ~(SR - 1), kWave);  // cs of the first row of i's slab
    if (Q % NTH == 0 || i < Q) {
      cs[i] = csv[n];
      dts[i] = dtv[n];
      ecs[i] = __expf(csv[n]);
      eslab[i] = __expf(csv[n] - csr);
    }
  }

  if constexpr (DMA) {
    __builtin_amdgcn_s_waitcnt(0x0070);  // this thread's copies of Gk have landed
    __syncthreads();                     // everyone's, and the per-token scalars
  }
  // state part of dxt^T: e_j (Gk B_j^T) with K = dstate
  f4 adx[NSLOT][TP];
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl)
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) adx[sl][tp] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NK; ++ks)
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) {
      Frag<T> gk;
      gfrag(gk, ks, tp);
#pragma unroll
      for (int sl = 0; sl < NSLOT; ++sl) mma(adx[sl][tp], gk, bfr[ks][sl]);
    }
  // <Gk, Hin>: waves 0 .. TP-1 of split 0 each cover Hin rows 16 w .. 16 w + 15
  float gh = 0.0f;
  if (gh_wave) {
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) {
      if (tp != wave) continue;
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        Frag<T> gk;
        gfrag(gk, ks, tp);
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) gh += frag_get(gk, s8) * frag_get(hf[ks], s8);
      }
    }
  }
  if constexpr (!DMA) slab_store(ra, DY0, W0);
  __syncthreads();

  const float cs_last = cs[Q - 1];
  const float Dh = Dp[h];
  // e_j scaling and q_j = dt_j <x_j, e_j B_j^T Gk>  (j = 16 J + c in this lane)
  float qsv[NSLOT], csv2[NSLOT], xdv[NSLOT];
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) {
    const int j = 16 * Js[sl] + c;
    const float e = __expf(cs_last - cs[j]);
    float qs = 0.0f;
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        adx[sl][tp][r] *= e;
        qs += adx[sl][tp][r] * frag_get(xf[sl][tp / 2], 4 * (tp & 1) + r);
      }
    }
    qsv[sl] = sum_q(qs) * dts[j];
  }

  float colsum[NSLOT];
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) colsum[sl] = 0.0f;
  float dd = 0.0f;

  if constexpr (DMA) {
    slab_dma(NS - 1, DY0, W0);
    if (NS >= 2) slab_dma(NS - 2, DY1, W1);
    if (NS >= 3) slab_dma(NS - 3, DY2, W2);
  }
  // slab s = NS - 1 - it, read from (dys, wts); (dyn, wtn) is the buffer the
  // slab PF ahead is copied into (DMA) or the next slab is stored into
  auto slab_step = [&](int it, T (*dys)[DPITCH], const TI* cbs, T (*dyn)[DPITCH], TI* cbn) {
    const int s = NS - 1 - it;
    if constexpr (DMA) {
      // slab s has landed once at most the copies of the min(PF - 1, s) slabs
      // issued after it are in flight (s_waitcnt vmcnt(n) lgkmcnt(0))
      const int younger = min(PF - 1, s);
      if (younger >= 2) __builtin_amdgcn_s_waitcnt(0x0070 | (2 * DPS));
      else if (younger == 1) __builtin_amdgcn_s_waitcnt(0x0070 | DPS);
      else __builtin_amdgcn_s_waitcnt(0x0070);
      // every thread's copies of slab s are in LDS, and the buffer copied into
      // next was last read in the previous step.  A plain s_barrier: the
      // workgroup fence of __syncthreads would also wait for the copies still
      // in flight.  The signal fences keep the compiler from moving LDS
      // accesses across it.
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (s - PF >= 0) slab_dma(s - PF, dyn, cbn);
    } else {
      if (it + 1 < NS) slab_load(ra, s - 1);
    }
    const int rb = 32 * s;  // first row of the slab

    // row sums of this slab's two row tiles (per lane: rows rb + 16 half + 4q + r)
    float rowtot[2][4];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int r = 0; r < 4; ++r) rowtot[half][r] = 0.0f;

    // dy^T operand tp of the slab (row p, chained K over its 32 rows), read
    // where it is used so that it holds no registers across the pair products
    auto fdt_load = [&](Frag<T>& f, int tp) {
      if constexpr (DSWZ) {  // rows 4q + c/4 and 16 below (same permutation)
        // lane c of a group receives headdim entry xrow(tp, c): the 4 lanes
        // addressing a row fetch the runs of 4 entries those columns need
        const int r0 = 4 * q + (c >> 2), col = XC ? 32 * (tp >> 1) + 8 * (c & 3) + 4 * (tp & 1) : 16 * tp + 4 * (c & 3);
        frag_load_kmajor_at(f, &dys[r0][dyc(r0, col)], &dys[r0 + 16][dyc(r0, col)]);
      } else {
        frag_load_kmajor<SR>(f, &dys[0][0], DPITCH, 0, 16 * tp, q, c);
      }
    };
    // dy row 16 half + c as a chained-K A fragment (K = headdim, from kp * 32)
    auto dy_row_frag = [&](Frag<T>& fd, int half, int kp) {
      const int yr = 16 * half + c;
      if constexpr (XC)
        frag_load(fd, &dys[yr][dyc(yr, kp * 32 + 8 * q)]);
      else if constexpr (DSWZ)
        frag_load2(fd, &dys[yr][dyc(yr, kp * 32 + 4 * q)], &dys[yr][dyc(yr, kp * 32 + 16 + 4 * q)]);
      else
        frag_load_chained<P>(fd, &dys[yr][0], kp * 32, q);
    };

    // intra-chunk pairs (I in this slab, J owned), I >= J.
    // Column tiles wholly before the slab ("full" pairs, the common case):
    // both row tiles lie after every column, so no mask is needed and the
    // decay factors at the slab's first row rb:
    //   Lam_ij = exp(cs_i - cs_rb) exp(cs_rb - cs_j),  both factors <= 1
    // (cs does not increase along the chunk).  Tiles J = 2s, 2s + 1 hold the
    // diagonal and take the masked direct form.
    f4 arow[2];                              // exp(cs_i - cs_rb), rows of this lane
#pragma unroll
    for (int half = 0; half < 2; ++half) arow[half] = *reinterpret_cast<const f4*>(&eslab[rb + 16 * half + 4 * q]);
    // W_ij = C_i . B_j of row tile 2s + half and owned column tile sl, in fp32
    // (lane (q, c): column j = 16 J + c, rows i = rb + 16 half + 4q + r)
    auto wtile = [&](f4& w, int half, int sl) {
      w = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        Frag<T> cf;
        staged_row_frag<N, NPC, CRPP>(cf, cbs, 16 * half + c, ks * 32 + 8 * q);
        mma(w, cf, bfr[ks][sl]);
      }
    };
    auto full_pair = [&](int sl) {
      const int cj = 16 * Js[sl] + c;
      const float bj = __expf(cs[rb] - cs[cj]);
      const float bdt = bj * dts[cj];
      f4 dp[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        dp[half] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kp = 0; kp < NKP; ++kp) {
          Frag<T> fd;
          dy_row_frag(fd, half, kp);
          mma(dp[half], fd, xf[sl][kp]);     // lane: column j = cj, rows i = rb + 16 half + 4q + r
        }
      }
      Frag<T> fa;                            // P[i][j] as the B operand (col j, K = i)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f4 wt;
        wtile(wt, half, sl);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float t = wt[r] * arow[half][r];
          frag_set<T>(fa, half * 4 + r, t * bj);
          const float rv = dp[half][r] * t * bdt;   // the same value enters both sums
          colsum[sl] += rv;
          rowtot[half][r] += rv;
        }
      }
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        Frag<T> fdt;
        fdt_load(fdt, tp);
        mma(adx[sl][tp], fdt, fa);
      }
    };
    // both owned column tiles full: every C and dy row fragment of the slab is
    // read once for the two tiles, half by half
    auto full_pairs2 = [&]() {
      float bj[2], bdt[2];
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const int cj = 16 * Js[sl] + c;
        bj[sl] = __expf(cs[rb] - cs[cj]);
        bdt[sl] = bj[sl] * dts[cj];
      }
      Frag<T> fa[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f4 wt[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          Frag<T> cf;
          staged_row_frag<N, NPC, CRPP>(cf, cbs, 16 * half + c, ks * 32 + 8 * q);
          mma(wt[0], cf, bfr[ks][0]);
          mma(wt[1], cf, bfr[ks][1]);
        }
        f4 dp[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kp = 0; kp < NKP; ++kp) {
          Frag<T> fd;
          dy_row_frag(fd, half, kp);
          mma(dp[0], fd, xf[0][kp]);
          mma(dp[1], fd, xf[1][kp]);
        }
#pragma unroll
        for (int sl = 0; sl < 2; ++sl)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float t = wt[sl][r] * arow[half][r];
            frag_set<T>(fa[sl], half * 4 + r, t * bj[sl]);
            const float rv = dp[sl][r] * t * bdt[sl];
            colsum[sl] += rv;
            rowtot[half][r] += rv;
          }
      }
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        Frag<T> fdt;
        fdt_load(fdt, tp);
        mma(adx[0][tp], fdt, fa[0]);
        mma(adx[1][tp], fdt, fa[1]);
      }
    };
    auto diag_pair = [&](int sl) {
      const int J = Js[sl];
      const int cj = 16 * J + c;             // lane's column j
      const float cs_cj = cs[cj];
      const float dt_cj = dts[cj];
      Frag<T> fa;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int I = 2 * s + half;
        if (I >= J) {
          f4 dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kp = 0; kp < NKP; ++kp) {
            Frag<T> fd;
            dy_row_frag(fd, half, kp);
            mma(dp, fd, xf[sl][kp]);
          }
          const int i0 = 16 * I + 4 * q;
          const f4 csi = *reinterpret_cast<const f4*>(&cs[i0]);
          f4 wt;
          wtile(wt, half, sl);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float lam = (i0 + r >= cj) ? __expf(csi[r] - cs_cj) : 0.0f;
            const float pv = wt[r] * lam;
            frag_set<T>(fa, half * 4 + r, pv);
            // the diagonal R_jj enters a row sum and a column sum with opposite
            // signs and cancels exactly, so it is left out of both
            const float rv = (i0 + r > cj) ? dp[r] * pv * dt_cj : 0.0f;
            colsum[sl] += rv;
            rowtot[half][r] += rv;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) frag_set<T>(fa, half * 4 + r, 0.0f);
        }
      }
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        Frag<T> fdt;
        fdt_load(fdt, tp);
        mma(adx[sl][tp], fdt, fa);
      }
    };
    if constexpr (NSLOT == 2) {
      const bool f0 = Js[0] < 2 * s, f1 = Js[1] < 2 * s;
      if (f0 && f1) full_pairs2();
      else if (f0) full_pair(0);
      else if (f1) full_pair(1);
    } else {
      if (Js[0] < 2 * s) full_pair(0);
    }
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl)
      if ((Js[sl] >> 1) == s) diag_pair(sl);

    {
      // the slab's 32 row totals of this wave: lane (q, c) ends with row
      // rb + 16 half + 4q + r, half = c / 8, r = (c / 2) % 4 (lanes c, c ^ 1 alike)
      float v8[8];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int r = 0; r < 4; ++r) v8[4 * half + r] = rowtot[half][r];
      rowacc[wave][rb + 16 * (c >> 3) + 4 * q + ((c >> 1) & 3)] = sum16_spread8(v8);
    }
    // next slab into the other buffer (its last readers passed the previous barrier)
    if constexpr (!DMA) {
      if (it + 1 < NS) slab_store(ra, dyn, cbn);
    }

    // column tiles whose rows are in this slab are complete: dx, <dxt_j, x_j>, column sums
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) {
      const int J = Js[sl];
      if ((J >> 1) != s) continue;
      const int j = 16 * J + c;
      csv2[sl] = sum_q(colsum[sl]);
      const float dtj = dts[j];
      float xd = 0.0f;
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        const V4 dv = *reinterpret_cast<const V4*>(
            &dys[j - rb][dyc(j - rb, XC ? 32 * (tp >> 1) + 8 * q + 4 * (tp & 1) : 16 * tp + 4 * q)]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float xv = frag_get(xf[sl][tp / 2], 4 * (tp & 1) + r);
          const float dyv = to_f(dv[r]);
          xd += adx[sl][tp][r] * xv;
          dd += dyv * xv;
          adx[sl][tp][r] = dtj * adx[sl][tp][r] + Dh * dyv;   // dx, stored after the loop
        }
      }
      xdv[sl] = sum_q(xd);
    }
    if constexpr (!DMA) __syncthreads();
  };
  if constexpr (DMA) {
    // every slab is its own copy of the step (NS <= 8), so each step's buffers
    // are fixed at compile time with no loop-carried state to merge
    static_assert(NS <= 8, "unrolled slab steps");
    slab_step(0, DY0, W0, DY3, W3);
    if constexpr (NS > 1) slab_step(1, DY1, W1, DY0, W0);
    if constexpr (NS > 2) slab_step(2, DY2, W2, DY1, W1);
    if constexpr (NS > 3) slab_step(3, DY3, W3, DY2, W2);
    if constexpr (NS > 4) slab_step(4, DY0, W0, DY3, W3);
    if constexpr (NS > 5) slab_step(5, DY1, W1, DY0, W0);
    if constexpr (NS > 6) slab_step(6, DY2, W2, DY1, W1);
    if constexpr (NS > 7) slab_step(7, DY3, W3, DY2, W2);
  } else {
    for (int it = 0; it < NS; it += 2) {
      slab_step(it, DY0, W0, DY1, W1);
      if (it + 1 < NS) slab_step(it + 1, DY1, W1, DY0, W0);
    }
  }

  // dx of the owned column tiles and their per-token sums
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) {
    const int j = 16 * Js[sl] + c;
    T* dxr = dx + ((row0 + j) * H + h) * P;
    if constexpr (XC) {
#pragma unroll
      for (int kp = 0; kp < TP / 2; ++kp) {
        V o;
#pragma unroll
        for (int r = 0; r < 8; ++r) o[r] = from_f<T>(adx[sl][2 * kp + r / 4][r % 4]);
        *reinterpret_cast<V*>(dxr + 32 * kp + 8 * q) = o;
      }
    } else {
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        V4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = from_f<T>(adx[sl][tp][r]);
        *reinterpret_cast<V4*>(dxr + 16 * tp + 4 * q) = o;
      }
    }
    if (q == 0) {
      part[NSPLIT * Q + j] = csv2[sl];
      part[(NSPLIT + 1) * Q + j] = qsv[sl];
      part[(NSPLIT + 2) * Q + j] = xdv[sl];
    }
  }

  // this split's row sums (fixed wave order) and scalars
  for (int i = threadIdx.x; i < Q; i += NTH) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += rowacc[w][i];
    part[split * Q + i] = v;
  }
  gh = wave_sum(gh);
  dd = wave_sum(dd);
  if (l == 0) { red[wave] = gh; red[NW + wave] = dd; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float ghs = 0.0f, dds = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) { ghs += red[w]; dds += red[NW + w]; }
    float* sc = dlscal + (int64_t)bkh * (NSPLIT + 1);
    if (split == 0) sc[0] = ghs;
    sc[1 + split] = dds;
  }
}

// ---------------------------------------------------------------------------
// The chunk-scan backward resident over heads (bf16 dy, chunk 256, headdim
// 64): one workgroup of 8 waves per (b, k, g) and slice of its heads, where
// k_chunk_scan_bwd takes one (b, k, h) per two workgroups and fetches the
// group's C rows (twice, as slabs) and the owned B rows again for every
// head.  Here the chunk's C rows stay in LDS and each wave's owned B_J
// fragments in registers for the whole slice; wave w owns the column tiles
// w and 15 - w (the zig-zag of k_chunk_scan_bwd, two per wave).  A head's
// dy rows and cs/dt travel global -> LDS by direct copies one head ahead
// (two buffers), its Gk into one buffer once every wave has formed the
// head's state term, and Hin (for <Gk, Hin>) and the owned x rows straight
// into registers during the previous head's epilogue.  The slab row
// factors exp(cs_i - cs_rb) are formed once per head into a small LDS
// table.  With the whole of dy in LDS the slab loop has no
// barrier; it runs from the chunk start, so a column tile is complete (and
// dx written) after the last slab.  The products are those of
// k_chunk_scan_bwd (W formed per slab in fp32 from the staged C rows), and
// so are the outputs: dx, and per token the row sums (all of them in the
// first split's row; k_dl_assemble then reads that row only), column sums,
// q_j and <dxt_j, x_j>, and per head <Gk, Hin> and <dy, x> (the first
// split's).
// Memory waits are explicit: the compiler takes copies into LDS and loads
// into registers for unordered on vmcnt and would wait for every copy in
// flight before a register's first use or an LDS store it cannot tell
// apart from a copy's destination.  So the head's top wait (vmcnt of the
// previous head's last stores) covers its copies, x and Hin, every path
// into it has issued the same stores, and the per-slab row sums and the
// row factors go to LDS through asm stores (published by an lgkmcnt(0)
// wait before the barrier that precedes their readers).
template <typename TI, int N>
__global__ __launch_bounds__(512, 1) void k_chunk_scan_bwd_heads(
    const TI* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ cs_g,
    const float* __restrict__ Dp, const TI* __restrict__ B, const TI* __restrict__ C, const bf16* __restrict__ hin,
    const bf16* __restrict__ gst, const bf16* __restrict__ dy, bf16* __restrict__ dx, float* __restrict__ dlpart,
    float* __restrict__ dlscal, const RowMap rm, int H, int G, int K, int hps, int nslice, int nbkg) {
  typedef bf16 T;
  constexpr int Q = 256, P = 64, NW = 8, NTH = NW * kWave;
  constexpr int NT = Q / 16, NS = NT / 2, TP = P / 16, NK = N / 32;
  constexpr int NSPLIT = scan_bwd_splits(Q);
  constexpr int EP = 16 / (int)sizeof(TI);
  constexpr int RBY = N * (int)sizeof(TI);
  constexpr int NPC = RBY / 16, CRPP = RBY >= 256 ? 1 : 256 / RBY;
  constexpr int GPC = N / 8;                        // 16-byte pieces of a Gk row
  constexpr int CPT = Q * NPC / NTH, DYPT = Q * P / 8 / NTH, GPT = P * N / 8 / NTH;
  constexpr int YST = 2 * (P / 32) + 2 * 2;         // dx stores and per-token writes per thread after the x loads
  static_assert(NT == 2 * NW && CPT * NTH == Q * NPC && DYPT * NTH * 8 == Q * P && GPT * NTH * 8 == P * N,
                "whole copies per thread");
  static_assert((NTH / NPC) % (CRPP * (NPC < 16 ? NPC : 16)) == 0 && (NTH / GPC) % GPC == 0 && (NTH / 8) % 16 == 0,
                "copy steps keep the row permutations");
  typedef typename Vec16<T>::type V;
  struct alignas(16) Buf {
    T DY[Q * P];                 // dy rows, pieces XOR-permuted by dyc
    float S[2 * Q + 4 * kWave];  // cs [0, Q), dt [Q, 2Q); the other waves' copies land past them, unread
  };
  __shared__ Buf B0, B1;
  __shared__ __attribute__((aligned(16))) TI CS[Q * N];  // the chunk's C rows, pieces XOR-permuted by row_swz
  __shared__ __attribute__((aligned(16))) T GS[P * N];   // Gk of the head, pieces of row r XOR-permuted by r mod GPC
  __shared__ float RA[NW][Q];                            // per-wave row sums of R
  __shared__ float RED[2 * NW];                          // per-wave <Gk, Hin> and <dy, x>
  __shared__ __attribute__((aligned(16))) float ES[Q];   // exp(cs_i - cs_rb) of the head, rb = first row of i's slab
  // dy rows in LDS: the 16-byte pieces of row r XOR-permuted by
  // f(r) = 4 (u mod 2) + u / 2, u = (r / 2) mod 8.  Within each row parity f
  // takes every value once over 16 rows, so a row fragment read (16
  // consecutive rows, one piece each) meets every bank once; and f(r) ^
  // f(r + 2) has bit 2 set, so the transposing dy^T reads (4 consecutive
  // rows, 4 pieces each) put rows r and r + 2 on disjoint pieces.
  auto dyf = [](int r) { return 4 * ((r >> 1) & 1) + ((r >> 2) & 3); };
  // storage column of dy element (r, col)
  auto dyc = [dyf](int r, int col) { return col ^ (8 * dyf(r)); };
  // headdim entry of row m of dxt^T tile tp (as in k_chunk_scan_bwd with bf16 and headdim 64)
  auto xrow = [](int tp, int m) { return 32 * (tp >> 1) + 8 * (m >> 2) + 4 * (tp & 1) + (m & 3); };

  const int xcd = blockIdx.x % 8, jb = blockIdx.x / 8;
  const int slice = jb % nslice, bkg = (jb / nslice) * 8 + xcd;
  if (bkg >= nbkg) return;  // whole workgroup, before any barrier
  const int g = bkg % G, bk = bkg / G, k = bk % K, b = bk / K;
  const int hpg = H / G, h0 = g * hpg + slice * hps, nh = min(hps, hpg - slice * hps);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t row0 = chunk_row0(rm, b, k, Q);
  x = rows_in(rm, k, x, rm.x);
  B = rows_in(rm, k, B, rm.B);
  C = rows_in(rm, k, C, rm.C);
  dy = rows_in(rm, k, dy, rm.dy);
  dx = rows_out(rm, k, dx, rm.dx);
  const int Js[2] = {wave, NT - 1 - wave};
  const int64_t rs = (int64_t)H * P;  // row stride of x / dy / dx

  // ---- the owned B fragments (K = dstate), and the chunk's C rows into LDS
  Frag<T> bfr[NK][2];
  {
    const int l = lane_id(), q = l >> 4, c = l & 15;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
        frag_load_k<N>(bfr[ks][sl], B + ((row0 + 16 * Js[sl] + c) * G + g) * N, ks * 32 + 8 * q);
    const int t = threadIdx.x, cr0 = t / NPC;
    const TI* cs0 = C + ((row0 + cr0) * G + g) * N + ((t % NPC) ^ row_swz<NPC, CRPP>(cr0)) * EP;
#pragma unroll
    for (int n = 0; n < CPT; ++n) lds_copy16(cs0 + (int64_t)n * (NTH / NPC) * G * N, &CS[(n * NTH + wave * kWave) * EP]);
  }
  // ---- one head's copies: dy and cs/dt into a buffer, Gk into GS.  Every
  // per-thread offset here and below is formed from a thread index passed
  // through an empty asm at each use, so the compiler forms it where it is
  // used instead of keeping it (as a 64-bit address) live over the head loop.
  auto tid = []() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
  };
  auto dma_dy = [&](int hh, Buf& Bn) {
    const int t = tid(), r = t / 8;
    const int h = h0 + hh;
    const T* dyh = dy + (row0 * H + h) * P;
    const uint32_t o = r * H * P + ((t % 8) ^ dyf(r)) * 8;
#pragma unroll
    for (int n = 0; n < DYPT; ++n)
      lds_copy16(dyh + (o + (uint32_t)(n * (NTH / 8) * H * P)), Bn.DY + (n * NTH + wave * kWave) * 8);
    const float* csb = cs_g + (((int64_t)b * H + h) * K + k) * Q;
    const float* dtb = dt + (((int64_t)b * H + h) * K + k) * Q;
    // wave 0 copies cs, wave 1 dt (a wave's 64 x 16 bytes each); the other
    // waves copy dt again into the spare tail, so every wave issues the
    // same copies
    static_assert(Q == 4 * kWave, "cs / dt: one wave's copy each");
    lds_copy16((wave == 0 ? csb : dtb) + 4 * (t % kWave), Bn.S + min(wave, 2) * kWave * 4);
  };
  auto dma_gk = [&](int hh) {
    const int t = tid(), r = t / GPC;
    const T* gh = gst + ((((int64_t)b * K + k) * H + h0 + hh) * P) * N;
    const uint32_t o = r * N + ((t % GPC) ^ (r & (GPC - 1))) * 8;
#pragma unroll
    for (int n = 0; n < GPT; ++n) lds_copy16(gh + (o + (uint32_t)(n * (NTH / GPC) * N)), &GS[(n * NTH + wave * kWave) * 8]);
  };

  // ---- row sums and scalars of head hh from the waves' shares (after a barrier)
  auto finish = [&](int hh) {
    const int t = tid();
    const int64_t bkh = ((int64_t)b * K + k) * H + h0 + hh;
    float* part = dlpart + bkh * dl_rows(Q) * Q;
    if (t < Q) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += RA[w][t];
      part[t] = v;  // the other split rows are not read after this kernel
    }
    if (t == 0) {
      float ghs = 0.0f, dds = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) { ghs += RED[w]; dds += RED[NW + w]; }
      float* sc = dlscal + bkh * (NSPLIT + 1);
      sc[0] = ghs;
      sc[1] = dds;
    }
  };
  auto barrier = [&]() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  // ---- head hh's register operands: x of the owned columns (lane (q, c): 8
  // consecutive headdim entries) and this thread's Hin pieces, matching the
  // GS pieces it reads for <Gk, Hin>.  Issued before the next head's copies,
  // so that waiting for them does not wait for those.
  typedef Frag<T> XF[2][2];
  typedef V HV[GPT];
  auto load_regs = [&](int hh, XF& xf, HV& hv) {
    int c = lane_id() & 15, q = lane_id() >> 4;
    asm volatile("" : "+v"(c), "+v"(q));
    const int t = tid();
    const int h = h0 + hh;
    const TI* xh = x + (row0 * H + h) * P;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int kp = 0; kp < 2; ++kp)
        frag_load(xf[sl][kp], xh + (uint32_t)((16 * Js[sl] + c) * H * P + kp * 32 + 8 * q));
    const T* hh0 = hin + (((int64_t)b * K + k) * H + h) * P * N;
#pragma unroll
    for (int n = 0; n < GPT; ++n) {
      const int u = n * NTH + t, r = u / GPC;
      hv[n] = *reinterpret_cast<const V*>(hh0 + (uint32_t)(r * N + ((u % GPC) ^ (r & (GPC - 1))) * 8));
    }
  };

  // ---- one head from buffer Bc
  auto head = [&](int hh, const Buf& Bc, const XF& xf, const HV& hv, XF& xn, HV& hn) {
    // The lane indices pass through an empty asm at every head, so the
    // addresses formed from them are formed here instead of being hoisted
    // out of the head loop.
    int c = lane_id() & 15, q = lane_id() >> 4;
    asm volatile("" : "+v"(c), "+v"(q));
    const int t = tid();
    const int h = h0 + hh;
    const float* cs = Bc.S;
    const float* dts = Bc.S + Q;
    const int64_t bkh = ((int64_t)b * K + k) * H + h;
    float* part = dlpart + bkh * dl_rows(Q) * Q;

    // state part of dxt^T: e_j (Gk B_j^T) with K = dstate (rows xrow(tp, .))
    f4 adx[2][TP];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) adx[sl][tp] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        const int r = xrow(tp, c);
        Frag<T> gk;
        frag_load(gk, &GS[r * N + ((((ks * 32 + 8 * q) / 8) ^ (r & (GPC - 1))) * 8)]);
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) mma(adx[sl][tp], gk, bfr[ks][sl]);
      }
    float gh = 0.0f;
#pragma unroll
    for (int n = 0; n < GPT; ++n) {
      const V a = *reinterpret_cast<const V*>(&GS[(n * NTH + t) * 8]);
#pragma unroll
      for (int e = 0; e < 8; ++e) gh += to_f(a[e]) * to_f(hv[n][e]);
    }
    // the slab row factors of this head (the previous head's slab loops are
    // done: they were before the last barrier)
    if (t < Q) {
      const float v = __expf(cs[t] - cs[t & ~31]);
      const uint32_t a = (uint32_t)(uintptr_t)&ES[t];
      asm volatile("ds_write_b32 %0, %1" : : "v"(a), "v"(v) : "memory");
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    barrier();  // every wave is done with GS (it takes the next head's Gk), ES is complete
    dma_gk(min(hh + 1, nh - 1));

    const float cs_last = cs[Q - 1];
    const float Dh = Dp[h];
    // e_j scaling and q_j = dt_j <x_j, e_j B_j^T Gk>  (j = 16 J + c in this lane)
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int j = 16 * Js[sl] + c;
      const float e = __expf(cs_last - cs[j]);
      float qs = 0.0f;
#pragma unroll
      for (int tp = 0; tp < TP; ++tp)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          adx[sl][tp][r] *= e;
          qs += adx[sl][tp][r] * frag_get(xf[sl][tp / 2], 4 * (tp & 1) + r);
        }
      qs = sum_q(qs) * dts[j];
      if (q == 0) part[(NSPLIT + 1) * Q + j] = qs;
    }

    float colsum[2] = {0.0f, 0.0f};
    // two slabs per iteration: their LDS addresses are one set of registers
    // with immediate offsets (measured 0.285 -> 0.276 ms on the 2.7B shape;
    // by four 0.280 ms, not unrolled 0.285 ms)
#pragma unroll 2
    for (int s = 0; s < NS; ++s) {
      const int rb = 32 * s;  // first row of the slab
      float rowtot[2][4];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int r = 0; r < 4; ++r) rowtot[half][r] = 0.0f;
      // dy^T operand tp of the slab (rows xrow(tp, .), chained K over its 32 rows)
      auto fdt_load = [&](Frag<T>& f, int tp) {
        const int r0 = rb + 4 * q + (c >> 2), col = 32 * (tp >> 1) + 8 * (c & 3) + 4 * (tp & 1);
        frag_load_kmajor_at(f, &Bc.DY[r0 * P + dyc(r0, col)], &Bc.DY[(r0 + 16) * P + dyc(r0, col)]);
      };
      // dy row rb + 16 half + c as an A fragment (K = headdim from kp * 32)
      auto dy_row_frag = [&](Frag<T>& fd, int half, int kp) {
        const int yr = rb + 16 * half + c;
        frag_load(fd, &Bc.DY[yr * P + dyc(yr, kp * 32 + 8 * q)]);
      };
      f4 arow[2];  // exp(cs_i - cs_rb), rows rb + 16 half + 4q + r of this lane
#pragma unroll
      for (int half = 0; half < 2; ++half) arow[half] = *reinterpret_cast<const f4*>(&ES[rb + 16 * half + 4 * q]);
      // W_ij = C_i . B_j of row tile 2s + half and owned column tile sl, in fp32
      auto wtile = [&](f4& w, int half, int sl) {
        w = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          Frag<T> cf;
          staged_row_frag<N, NPC, CRPP>(cf, CS, rb + 16 * half + c, ks * 32 + 8 * q);
          mma(w, cf, bfr[ks][sl]);
        }
      };
      // column tiles wholly before the slab: the decay factors at the slab's first row
      auto full_pair = [&](int sl) {
        const int cj = 16 * Js[sl] + c;
        const float bj = __expf(cs[rb] - cs[cj]);
        const float bdt = bj * dts[cj];
        f4 dp[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          dp[half] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kp = 0; kp < 2; ++kp) {
            Frag<T> fd;
            dy_row_frag(fd, half, kp);
            mma(dp[half], fd, xf[sl][kp]);
          }
        }
        Frag<T> fa;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          f4 wt;
          wtile(wt, half, sl);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float tv = wt[r] * arow[half][r];
            frag_set<T>(fa, half * 4 + r, tv * bj);
            const float rv = dp[half][r] * tv * bdt;
            colsum[sl] += rv;
            rowtot[half][r] += rv;
          }
        }
#pragma unroll
        for (int tp = 0; tp < TP; ++tp) {
          Frag<T> fdt;
          fdt_load(fdt, tp);
          mma(adx[sl][tp], fdt, fa);
        }
      };
      auto full_pairs2 = [&]() {
        float bj[2], bdt[2];
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          const int cj = 16 * Js[sl] + c;
          bj[sl] = __expf(cs[rb] - cs[cj]);
          bdt[sl] = bj[sl] * dts[cj];
        }
        Frag<T> fa[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          f4 wt[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
          for (int ks = 0; ks < NK; ++ks) {
            Frag<T> cf;
            staged_row_frag<N, NPC, CRPP>(cf, CS, rb + 16 * half + c, ks * 32 + 8 * q);
            mma(wt[0], cf, bfr[ks][0]);
            mma(wt[1], cf, bfr[ks][1]);
          }
          f4 dp[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
          for (int kp = 0; kp < 2; ++kp) {
            Frag<T> fd;
            dy_row_frag(fd, half, kp);
            mma(dp[0], fd, xf[0][kp]);
            mma(dp[1], fd, xf[1][kp]);
          }
#pragma unroll
          for (int sl = 0; sl < 2; ++sl)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float tv = wt[sl][r] * arow[half][r];
              frag_set<T>(fa[sl], half * 4 + r, tv * bj[sl]);
              const float rv = dp[sl][r] * tv * bdt[sl];
              colsum[sl] += rv;
              rowtot[half][r] += rv;
            }
        }
#pragma unroll
        for (int tp = 0; tp < TP; ++tp) {
          Frag<T> fdt;
          fdt_load(fdt, tp);
          mma(adx[0][tp], fdt, fa[0]);
          mma(adx[1][tp], fdt, fa[1]);
        }
      };
      // the slab holding column tile J's own rows: the masked direct form
      auto diag_pair = [&](int sl) {
        const int J = Js[sl];
        const int cj = 16 * J + c;
        const float cs_cj = cs[cj];
        const float dt_cj = dts[cj];
        Frag<T> fa;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int I = 2 * s + half;
          if (I >= J) {
            f4 dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) {
              Frag<T> fd;
              dy_row_frag(fd, half, kp);
              mma(dp, fd, xf[sl][kp]);
            }
            const int i0 = 16 * I + 4 * q;
            const f4 csi = *reinterpret_cast<const f4*>(&cs[i0]);
            f4 wt;
            wtile(wt, half, sl);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float lam = (i0 + r >= cj) ? __expf(csi[r] - cs_cj) : 0.0f;
              const float pv = wt[r] * lam;
              frag_set<T>(fa, half * 4 + r, pv);
              // the diagonal R_jj cancels between the row and column sums and is left out of both
              const float rv = (i0 + r > cj) ? dp[r] * pv * dt_cj : 0.0f;
              colsum[sl] += rv;
              rowtot[half][r] += rv;
            }
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) frag_set<T>(fa, half * 4 + r, 0.0f);
          }
        }
#pragma unroll
        for (int tp = 0; tp < TP; ++tp) {
          Frag<T> fdt;
          fdt_load(fdt, tp);
          mma(adx[sl][tp], fdt, fa);
        }
      };
      {
        const bool f0 = Js[0] < 2 * s, f1 = Js[1] < 2 * s;
        if (f0 && f1) full_pairs2();
        else if (f0) full_pair(0);
        else if (f1) full_pair(1);
      }
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
        if ((Js[sl] >> 1) == s) diag_pair(sl);
      // the slab's 32 row totals of this wave: lane (q, c) ends with row
      // rb + 16 half + 4q + r, half = c / 8, r = (c / 2) % 4 (lanes c, c ^ 1 alike)
      float v8[8];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int r = 0; r < 4; ++r) v8[4 * half + r] = rowtot[half][r];
      {
        const float v = sum16_spread8(v8);
        const uint32_t a = (uint32_t)(uintptr_t)&RA[wave][rb + 16 * (c >> 3) + 4 * q + ((c >> 1) & 3)];
        asm volatile("ds_write_b32 %0, %1" : : "v"(a), "v"(v) : "memory");
      }
    }

    // the next head's x and Hin, in flight over this head's epilogue and the
    // head switch (the last head reloads its own)
    load_regs(min(hh + 1, nh - 1), xn, hn);

    // the owned columns are complete: <dxt_j, x_j>, <dy_j, x_j>, dx, the per-token sums
    float dd = 0.0f;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      // x passes through an empty asm here, so that its fp32 values for q_j
      // are converted again instead of being held over the slab loop
      Frag<T> xe[2] = {xf[sl][0], xf[sl][1]};
      asm volatile("" : "+v"(xe[0].v), "+v"(xe[1].v));
      const int j = 16 * Js[sl] + c;
      const float dtj = dts[j];
      float xd = 0.0f;
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        const typename Vec4<T>::type dv = *reinterpret_cast<const typename Vec4<T>::type*>(
            &Bc.DY[j * P + dyc(j, 32 * (tp >> 1) + 8 * q + 4 * (tp & 1))]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float xv = frag_get(xe[tp / 2], 4 * (tp & 1) + r);
          const float dyv = to_f(dv[r]);
          xd += adx[sl][tp][r] * xv;
          dd += dyv * xv;
          adx[sl][tp][r] = dtj * adx[sl][tp][r] + Dh * dyv;
        }
      }
      const float csv = sum_q(colsum[sl]);
      const float xdv = sum_q(xd);
      T* dxr = dx + ((row0 + j) * H + h) * P;
#pragma unroll
      for (int kp = 0; kp < TP / 2; ++kp) {
        V o;
#pragma unroll
        for (int r = 0; r < 8; ++r) o[r] = from_f<T>(adx[sl][2 * kp + r / 4][r % 4]);
        *reinterpret_cast<V*>(dxr + 32 * kp + 8 * q) = o;
      }
      // the four lanes of column j hold the same sums and all store them:
      // no branch, so every path from the x loads above to the next head's
      // wait issues the same stores
      part[NSPLIT * Q + j] = csv;
      part[(NSPLIT + 2) * Q + j] = xdv;
    }
    gh = wave_sum(gh);
    dd = wave_sum(dd);
    if (lane_id() == 0) {
      RED[wave] = gh;
      RED[NW + wave] = dd;
    }
  };

  // ---- heads.  Head hh's dy and cs/dt live in buffer hh & 1, its Gk in GS,
  // its x and Hin in registers loaded during the previous head.  At the top
  // of a head its copies and loads have landed once at most the previous
  // head's dx and per-token stores (issued after the last of them, the x and
  // Hin loads) are in flight; after the barrier the other buffer is free,
  // and the previous head's row sums are complete.  The wait and barrier
  // are unconditional (the first head has nothing in flight), so that every
  // path into a head has waited the same.  Unrolled by two so that every
  // LDS access names its buffer.
  XF xa, xb;
  HV ha, hb;
  load_regs(0, xa, ha);
  dma_dy(0, B0);
  dma_gk(0);
  __builtin_amdgcn_s_waitcnt(0x0070);  // C rows, B fragments, head 0
  __syncthreads();
  // head 0's registers pass through an empty asm here, so their loads are
  // issued (and waited for) before this point: the loop's first wait then
  // finds them complete on every path into it
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) asm volatile("" : "+v"(xa[sl][0].v), "+v"(xa[sl][1].v));
#pragma unroll
  for (int n = 0; n < GPT; ++n) asm volatile("" : "+v"(ha[n]));
  auto step = [&](int hh, const Buf& Bc, Buf& Bn, const XF& xc, const HV& hc, XF& xn, HV& hn) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(YST));
    barrier();
    if (hh > 0) finish(hh - 1);
    dma_dy(min(hh + 1, nh - 1), Bn);
    head(hh, Bc, xc, hc, xn, hn);
  };
  for (int hh = 0; hh < nh; hh += 2) {
    step(hh, B0, B1, xa, ha, xb, hb);
    if (hh + 1 < nh) step(hh + 1, B1, B0, xb, hb, xa, ha);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));  // the last head's spare copies too
  __syncthreads();
  finish(nh - 1);
}

// dl, ddt and the chunk's dA / dD partials from the per-token partial sums of
// k_chunk_scan_bwd and (the state-to-output term t_i, in ntp headdim-tile
// shares) of the chunk-state gradient:
//   dl_j = sum_{i >= j} (row sum_i + t_i - column sum_i)  [suffix sum]
//        + sum_{j' < j} q_j'                          [exclusive prefix sum]
//        + exp(cs_{Q-1}) <Gk, Hin_k>
// (the q terms, added at the chunk end and subtracted at each token, are
// summed directly as a prefix so no large terms cancel), then
//   ddt_j = A dl_j + <dxt_j, x_j>,  dA partial = sum_j dt_j dl_j.
// One wave per (b, k, h) and 4 heads per workgroup (b K H / 4 workgroups, so
// the launch fills the chip); lane l owns the Q / 64 consecutive tokens
// starting at l Q / 64.  A chunk's head groups share the token rows of ddt
// (one step per head), so its workgroups are dealt 8 dispatch slots apart:
// one XCD's L2 gathers each row's heads before it goes to memory.
template <typename T, int Q, int NTP, int NSP>
__global__ __launch_bounds__(256) void k_dl_assemble(const float* __restrict__ dlpart, const float* __restrict__ dlscal,
                                                     const float* __restrict__ cs_g, const float* __restrict__ dt,
                                                     const float* __restrict__ Ap, T* __restrict__ ddt,
                                                     float* __restrict__ dapart, float* __restrict__ ddpart,
                                                     float* __restrict__ dbiaspart, const RowMap rm, int H, int K,
                                                     int softplus, int nbk) {
  // NTP: headdim-tile shares of the state-to-output term; NSP: split rows
  // holding row sums (the layout has NSPLIT).  Both fixed at compile time,
  // so every load of a lane is issued before the first wait.
  constexpr int NSPLIT = scan_bwd_splits(Q);
  static_assert(NSP >= 1 && NSP <= NSPLIT && NTP >= 1, "rows");
  constexpr int HPB = 4;                      // heads (waves) per workgroup
  constexpr int TPL = Q / kWave;
  static_assert(Q % kWave == 0, "chunk");
  const int nhb = (H + HPB - 1) / HPB;
  const int xcd = blockIdx.x % 8, jb = blockIdx.x / 8;
  const int hb = jb % nhb, bk = (jb / nhb) * 8 + xcd;
  if (bk >= nbk) return;  // whole workgroup; no barrier in this kernel
  const int k = bk % K, b = bk / K;
  const int jl = lane_id();
  const int h = HPB * hb + threadIdx.x / kWave;
  if (h >= H) return;  // whole wave; no barrier in this kernel
  const int bkh = bk * H + h;
  const int64_t row0 = chunk_row0(rm, b, k, Q);
  const float* dtc = dt + (((int64_t)b * H + h) * K + k) * Q;
  ddt = rows_out(rm, k, ddt, rm.ddt);
  const float* part = dlpart + (int64_t)bkh * dl_rows(Q) * Q;
  const float* sc = dlscal + (int64_t)bkh * (NSPLIT + 1);
  const float* csc = cs_g + (((int64_t)b * H + h) * K + k) * Q;
  // the per-head values first (uniform: scalar loads), with the lane's rows below
  const float cs_last = csc[Q - 1], ghin = sc[0], Ah = Ap[h];
  float dds = 0.0f;
#pragma unroll
  for (int sp = 0; sp < NSP; ++sp) dds += sc[1 + sp];
  const int j0 = jl * TPL;
  float v[TPL], qp[TPL], dtv[TPL], xdv[TPL];
#pragma unroll
  for (int t = 0; t < TPL; ++t) {
    dtv[t] = dtc[j0 + t];
    xdv[t] = part[(NSPLIT + 2) * Q + j0 + t];
    float rs = part[j0 + t];
#pragma unroll
    for (int sp = 1; sp < NSP; ++sp) rs += part[sp * Q + j0 + t];
    float ts = part[(NSPLIT + 3) * Q + j0 + t];
#pragma unroll
    for (int tp = 1; tp < NTP; ++tp) ts += part[(NSPLIT + 3 + tp) * Q + j0 + t];
    v[t] = (rs + ts) - part[NSPLIT * Q + j0 + t];
    qp[t] = part[(NSPLIT + 1) * Q + j0 + t];
  }
#pragma unroll
  for (int t = TPL - 2; t >= 0; --t) v[t] += v[t + 1];
  float qrun = 0.0f;  // exclusive prefix of q inside this lane's tokens
#pragma unroll
  for (int t = 0; t < TPL; ++t) {
    const float qt = qp[t];
    qp[t] = qrun;
    qrun += qt;
  }
  // across the wave: suffix of the lane sums v[0], prefix of qrun
  float incl = v[0], qincl = qrun;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float o = __shfl_down(incl, off, kWave);
    if (jl + off < kWave) incl += o;
    const float p = __shfl_up(qincl, off, kWave);
    if (jl >= off) qincl += p;
  }
  float excl = __shfl_down(incl, 1, kWave);
  if (jl == kWave - 1) excl = 0.0f;
  const float qexcl = qincl - qrun;
  const float tail = __expf(cs_last) * ghin;
  float da = 0.0f, dbias = 0.0f;
#pragma unroll
  for (int t = 0; t < TPL; ++t) {
    const int j = j0 + t;
    const float dl = v[t] + excl + (qp[t] + qexcl) + tail;
    da += dtv[t] * dl;
    float g = Ah * dl + xdv[t];
    if (softplus) {
      // the step was softplus(z): d dt / dz = sigmoid(z) = 1 - exp(-dt)
      g *= -expm1f(-dtv[t]);
      dbias += g;
    }
    ddt[(row0 + j) * H + h] = from_f<T>(g);
  }
  da = wave_sum(da);
  if (softplus) dbias = wave_sum(dbias);
  if (jl == 0) {
    dapart[bkh] = da;
    ddpart[bkh] = dds;
    if (softplus) dbiaspart[bkh] = dbias;
  }
}

// ---------------------------------------------------------------------------
// Head-summed masked outer products for one (b, k, g) and one 64x64 block
// (IB, JB), JB <= IB, of the chunk's Q x Q matrix:
//   dW_ij = sum_{h in g} <dy_i, xt_j> exp(cs_i - cs_j)   (j <= i, else 0)
// Off-diagonal blocks (IB > JB): every i lies after every j, so with the
// reference token r = 64 JB + 63 (last of block JB) the decay splits as
// exp(cs_i - cs_r) exp(cs_r - cs_j), both factors <= 1; the row factor goes
// onto the dy fragments in registers and the column factor (with dt_j) onto
// the x rows as they are staged, so dW_IJ is one product with K = (head,
// headdim) accumulated on the matrix cores across heads.  Diagonal blocks
// multiply each head's product by the masked decay element-wise.
// Wave w owns the block's rows 16w .. 16w + 15: their dy fragments come
// straight from global memory (K = headdim is contiguous there); the head's
// 64 x rows are staged row-major in LDS once per workgroup (double-buffered,
// the next head is loaded into registers while the current one is used).
// A slice of hps heads of the group is summed per workgroup; each slice
// writes its own partial dW (summed later in a fixed order).
constexpr int DW_DEPTH = 2;  // heads in flight per dW workgroup (3 measured no faster, 4 slower)

template <typename T, int P>
struct DwLds {
  static constexpr int XP = P + 16 / sizeof(T);  // row pitch of the staged x rows
  __attribute__((aligned(16))) T Xs[2][64][XP];
  __attribute__((aligned(16))) float csJ[2][64];  // diagonal blocks: cs_j, dt_j of the staged head
  __attribute__((aligned(16))) float dtJ[2][64];
};

template <typename T, typename TI, int Q, int P, bool DIAG>
__device__ __forceinline__ void dw_block(const TI* __restrict__ x, const float* __restrict__ dt,
                                         const float* __restrict__ cs_g, const T* __restrict__ dy,
                                         float* __restrict__ dw, const RowMap& rm, int H, int G, int K, int hps,
                                         int bkg, int nbkg, int slice, int IB, int JB, DwLds<T, P>& sm, int dw_st) {
  constexpr int NTH = 256;
  constexpr int NKP = (P + 31) / 32;
  constexpr int XP = DwLds<T, P>::XP;
  constexpr int VN = Vec16<T>::n;
  constexpr int XPIECES = 64 * P / VN;
  constexpr int XPT = (XPIECES + NTH - 1) / NTH;
  typedef typename Vec16<T>::type V;
  auto& Xs = sm.Xs;
  auto& csJ = sm.csJ;
  auto& dtJ = sm.dtJ;

  const int g = bkg % G, bk = bkg / G, k = bk % K, b = bk / K;
  const int wave = threadIdx.x / kWave, l = lane_id(), q = l >> 4, c = l & 15;
  const int64_t row0 = chunk_row0(rm, b, k, Q);
  x = rows_in(rm, k, x, rm.x);
  dy = rows_in(rm, k, dy, rm.dy);
  const int hpg = H / G;
  const int h0 = g * hpg + slice * hps;                       // first head of this slice
  const int nh = min(hps, hpg - slice * hps);                 // heads in this slice
  const int i0 = 64 * IB, j0 = 64 * JB, ref = j0 + 63;
  const int ia = i0 + 16 * wave + c;                          // this lane's row (A operand)

  // DW_DEPTH heads in flight, in a ring of register sets: a set holds the raw
  // loads of one head (x rows, and the step / cumsum values its factors come
  // from), and the exponentials are taken only when the head is staged or
  // used, so no load is waited for before its head's turn.  Head indices past
  // the slice are clamped (a repeated load) so the loads carry no branch.
  struct HeadRegs {
    V xv[XPT];
    float dtv[XPT], csv[XPT];          // off-diagonal: dt_j, cs_j of the staged x rows
    Frag<T> av[NKP];                   // dy fragments of this wave's rows
    float cref, cia, jcs, jdt, csi[4];
  };
  HeadRegs R[DW_DEPTH];
  auto load = [&](HeadRegs& R, int hh) {
    const int h = h0 + min(hh, nh - 1);
    const float* csb = cs_g + (((int64_t)b * H + h) * K + k) * Q;
    const float* dtb = dt + (((int64_t)b * H + h) * K + k) * Q;
#pragma unroll
    for (int n = 0; n < XPT; ++n) {
      const int u = threadIdx.x + NTH * n;
      if (XPIECES % NTH == 0 || u < XPIECES) {
        const int r = u / (P / VN);
        R.xv[n] = load_vec16<T, TI>(x + ((row0 + j0 + r) * H + h) * P + (u % (P / VN)) * VN);
        if (!DIAG) {
          R.dtv[n] = dtb[j0 + r];
          R.csv[n] = csb[j0 + r];
        }
      }
    }
    const T* arow = dy + ((row0 + ia) * H + h) * P;
#pragma unroll
    for (int kp = 0; kp < NKP; ++kp) frag_load_chained<P>(R.av[kp], arow, kp * 32, q);
    if (!DIAG) {
      R.cref = csb[ref];
      R.cia = csb[ia];
    } else {
      const int jl = threadIdx.x & 63;   // threads 0..63 stage cs_j, dt_j
      R.jcs = csb[j0 + jl];
      R.jdt = dtb[j0 + jl];
#pragma unroll
      for (int r = 0; r < 4; ++r) R.csi[r] = csb[i0 + 16 * wave + 4 * q + r];
    }
  };
  auto store = [&](const HeadRegs& R, int bf) {
#pragma unroll
    for (int n = 0; n < XPT; ++n) {
      const int u = threadIdx.x + NTH * n;
      if (XPIECES % NTH == 0 || u < XPIECES) {
        T* d = &Xs[bf][u / (P / VN)][(u % (P / VN)) * VN];
        if (DIAG) {
          *reinterpret_cast<V*>(d) = R.xv[n];
        } else {
          const float xs = R.dtv[n] * __expf(R.cref - R.csv[n]);
          V w;
#pragma unroll
          for (int e = 0; e < VN; ++e) w[e] = from_f<T>(to_f(R.xv[n][e]) * xs);
          *reinterpret_cast<V*>(d) = w;
        }
      }
    }
    if (DIAG && threadIdx.x < 64) {
      csJ[bf][threadIdx.x] = R.jcs;
      dtJ[bf][threadIdx.x] = R.jdt;
    }
  };

  f4 acc[4];
#pragma unroll
  for (int tj = 0; tj < 4; ++tj) acc[tj] = f4{0.f, 0.f, 0.f, 0.f};
  // head hh: its set cur was loaded DW_DEPTH heads earlier; nxt holds head hh + 1
  auto step = [&](HeadRegs& cur, HeadRegs& nxt, int hh) {
    const int bf = hh & 1;
    const float ascale = DIAG ? 1.0f : __expf(cur.cia - cur.cref);
    Frag<T> fa[NKP];
#pragma unroll
    for (int kp = 0; kp < NKP; ++kp)
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8)
        frag_set<T>(fa[kp], s8, DIAG ? frag_get(cur.av[kp], s8) : frag_get(cur.av[kp], s8) * ascale);
    float csi[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) csi[r] = cur.csi[r];
    __syncthreads();  // head hh is in buffer bf; buffer bf ^ 1 is no longer read
    load(cur, hh + DW_DEPTH);
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      if (DIAG && tj > wave) continue;  // strictly above the diagonal: zero
      f4 dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kp = 0; kp < NKP; ++kp) {
        Frag<T> fb;
        frag_load_chained<P>(fb, &Xs[bf][16 * tj + c][0], kp * 32, q);
        if (DIAG) mma(dp, fa[kp], fb);
        else mma(acc[tj], fa[kp], fb);
      }
      if (DIAG) {
        const int jl = 16 * tj + c;
        const float csj = csJ[bf][jl], dtj = dtJ[bf][jl];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int il = 16 * wave + 4 * q + r;
          const float lam = (il >= jl) ? __expf(csi[r] - csj) : 0.0f;
          acc[tj][r] += dp[r] * dtj * lam;
        }
      }
    }
    store(nxt, bf ^ 1);  // head hh + 1 (a repeat past the slice, never read)
  };
#pragma unroll
  for (int d = 0; d < DW_DEPTH; ++d) load(R[d], d);
  store(R[0], 0);
  for (int hh = 0; hh < nh; hh += DW_DEPTH) {
#pragma unroll
    for (int d = 0; d < DW_DEPTH; ++d)
      if (hh + d < nh) step(R[d], R[(d + 1) % DW_DEPTH], hh + d);
  }
  // dw_st: a single head slice, stored in the storage dtype (the rounding the
  // dC/dB products apply to it anyway), else float32 per-slice partials
  if (dw_st) {
    T* o = reinterpret_cast<T*>(dw) + (int64_t)bkg * Q * Q;
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      const int j = j0 + 16 * tj + c;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[(int64_t)(i0 + 16 * wave + 4 * q + r) * Q + j] = from_f<T>(acc[tj][r]);
    }
  } else {
    float* o = dw + ((int64_t)slice * nbkg + bkg) * Q * Q;
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      const int j = j0 + 16 * tj + c;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[(int64_t)(i0 + 16 * wave + 4 * q + r) * Q + j] = acc[tj][r];
    }
  }
}

// ---------------------------------------------------------------------------
// Head sums of dC / dB for one (b, k, g), one 64-row block RB of the chunk
// and one slice of hps heads:
//   dC: part[i][n] = sum_{h in slice} exp(cs_i) sum_p dy_i[p] Hin_k[p][n]
//   dB: part[j][n] = sum_{h in slice} e_j dt_j  sum_p x_j[p]  Gk[p][n]
// One product per head with K = headdim on the matrix cores.  Each wave
// owns 16 rows: their dy (or x) fragments come straight from global memory
// (K = headdim is contiguous there) and take the row's scale in registers;
// the head's state is staged row-major in LDS (double-buffered, the next
// head is loaded into registers while the current one is used) and read
// K-major with the transposing LDS read.  Every slice writes an fp32
// partial; k_bc_final adds the slices and the dW part.
template <typename T, int P, int N>
struct BcLds {
  static constexpr int SP = N + 16;  // state row pitch (8 mod 16 dwords for N = 64, 128)
  __attribute__((aligned(16))) T Ss[2][P][SP];
};

template <typename T, typename TI, int Q, int P, int N, bool DB>
__device__ __forceinline__ void bc_heads_block(const TI* __restrict__ x, const float* __restrict__ dt,
                                               const float* __restrict__ cs_g, const T* __restrict__ dy,
                                               const T* __restrict__ state, float* __restrict__ out,
                                               const RowMap& rm, int H, int G, int K, int hps, int bkg, int nbkg,
                                               int slice, int RB, BcLds<T, P, N>& sm) {
  constexpr int NTH = 256;
  constexpr int TN = N / 16, NKP = (P + 31) / 32;
  constexpr int VN = Vec16<T>::n;
  constexpr int SP = BcLds<T, P, N>::SP;
  constexpr int SPIECES = P * N / VN;
  constexpr int SPT = (SPIECES + NTH - 1) / NTH;
  static_assert(P == 16 || P % 32 == 0, "headdim");
  typedef typename Vec16<T>::type V;
  auto& Ss = sm.Ss;

  const int g = bkg % G, bk = bkg / G, k = bk % K, b = bk / K;
  const int wave = threadIdx.x / kWave, l = lane_id(), q = l >> 4, c = l & 15;
  const int64_t row0 = chunk_row0(rm, b, k, Q);
  x = rows_in(rm, k, x, rm.x);
  dy = rows_in(rm, k, dy, rm.dy);
  const int64_t prow0 = ((int64_t)b * K + k) * Q;  // row of the fp32 partials (chunk rows)
  const int hpg = H / G;
  const int h0 = g * hpg + slice * hps;
  const int nh = min(hps, hpg - slice * hps);
  const int i = 64 * RB + 16 * wave + c;     // this lane's row (A operand)

  // registers of the head in flight
  V sv[SPT];
  Frag<T> av[NKP];
  float ascale = 0.0f;
  auto load = [&](int hh) {
    const int h = h0 + hh;
    const T* st = state + (((int64_t)b * K + k) * H + h) * P * N;
#pragma unroll
    for (int n = 0; n < SPT; ++n) {
      const int u = threadIdx.x + NTH * n;
      if (SPIECES % NTH == 0 || u < SPIECES) sv[n] = *reinterpret_cast<const V*>(st + u * VN);
    }
    if constexpr (DB) {
      const TI* urow = x + ((row0 + i) * H + h) * P;
#pragma unroll
      for (int kp = 0; kp < NKP; ++kp) frag_load_chained<P>(av[kp], urow, kp * 32, q);
    } else {
      const T* urow = dy + ((row0 + i) * H + h) * P;
#pragma unroll
      for (int kp = 0; kp < NKP; ++kp) frag_load_chained<P>(av[kp], urow, kp * 32, q);
    }
    const float* csb = cs_g + (((int64_t)b * H + h) * K + k) * Q;
    ascale = DB ? __expf(csb[Q - 1] - csb[i]) * dt[(((int64_t)b * H + h) * K + k) * Q + i] : __expf(csb[i]);
  };
  auto store = [&](int bf) {
#pragma unroll
    for (int n = 0; n < SPT; ++n) {
      const int u = threadIdx.x + NTH * n;
      if (SPIECES % NTH == 0 || u < SPIECES) *reinterpret_cast<V*>(&Ss[bf][u / (N / VN)][(u % (N / VN)) * VN]) = sv[n];
    }
  };

  f4 acc[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) acc[tn] = f4{0.f, 0.f, 0.f, 0.f};

  load(0);
  store(0);
  for (int hh = 0; hh < nh; ++hh) {
    const int bf = hh & 1;
    // the current head's row fragments, scaled
    Frag<T> fa[NKP];
#pragma unroll
    for (int kp = 0; kp < NKP; ++kp)
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) frag_set<T>(fa[kp], s8, frag_get(av[kp], s8) * ascale);
    __syncthreads();  // head hh is in buffer bf; buffer bf ^ 1 is no longer read
    if (hh + 1 < nh) load(hh + 1);
#pragma unroll
    for (int kp = 0; kp < NKP; ++kp) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        Frag<T> fb;
        frag_load_kmajor<P>(fb, &Ss[bf][0][0], SP, kp * 32, 16 * tn, q, c);
        mma(acc[tn], fa[kp], fb);
      }
    }
    if (hh + 1 < nh) store(bf ^ 1);
  }
  float* o = out + (int64_t)slice * nbkg * Q * N;  // slice stride b*K*G*Q*N
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 64 * RB + 16 * wave + 4 * q + r;
      o[((prow0 + row) * G + g) * N + 16 * tn + c] = acc[tn][r];
    }
  }
}

// Every group-level head sum of the backward in one launch: per work item
// ((b, k, g), head slice) the Q/64 row blocks of the dC and of the dB head
// sums and the Q/64 (Q/64 + 1)/2 blocks of dW.  All of them read the same
// dy and x rows of the item's heads (and walk the heads in the same order),
// and the blocks of one item are dealt to workgroups 8 dispatch slots apart,
// which the round-robin dispatch over the 8 XCDs places on one XCD at about
// the same time: the rows come from HBM once and from that XCD's L2 for the
// other blocks.  The heavier head-sum blocks come first in an item.
template <typename T, typename TI, int Q, int P, int N>
__global__ __launch_bounds__(256) void k_dw_heads(const TI* __restrict__ x, const float* __restrict__ dt,
                                                  const float* __restrict__ cs_g, const T* __restrict__ dy,
                                                  const T* __restrict__ hin, const T* __restrict__ gst,
                                                  float* __restrict__ dw, float* __restrict__ dcpart,
                                                  float* __restrict__ dbpart, const RowMap rm, int H, int G, int K,
                                                  int hps, int nbkg, int nitems, int dw_st) {
  constexpr int NB = Q / 64, NBLK = 2 * NB + NB * (NB + 1) / 2;
  constexpr size_t LDS = sizeof(DwLds<T, P>) > sizeof(BcLds<T, P, N>) ? sizeof(DwLds<T, P>) : sizeof(BcLds<T, P, N>);
  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS];
  const int xcd = blockIdx.x % 8, j = blockIdx.x / 8;
  const int blk = j % NBLK, item = (j / NBLK) * 8 + xcd;
  if (item >= nitems) return;  // whole workgroup, before any barrier
  const int bkg = item % nbkg, slice = item / nbkg;
  if (blk < NB) {
    bc_heads_block<T, TI, Q, P, N, false>(x, dt, cs_g, dy, hin, dcpart, rm, H, G, K, hps, bkg, nbkg, slice, blk,
                                      *reinterpret_cast<BcLds<T, P, N>*>(smem));
  } else if (blk < 2 * NB) {
    bc_heads_block<T, TI, Q, P, N, true>(x, dt, cs_g, dy, gst, dbpart, rm, H, G, K, hps, bkg, nbkg, slice, blk - NB,
                                     *reinterpret_cast<BcLds<T, P, N>*>(smem));
  } else if (blk < 3 * NB) {
    const int d = blk - 2 * NB;
    dw_block<T, TI, Q, P, true>(x, dt, cs_g, dy, dw, rm, H, G, K, hps, bkg, nbkg, slice, d, d,
                            *reinterpret_cast<DwLds<T, P>*>(smem), dw_st);
  } else {
    const int y = blk - 3 * NB;  // pairs IB > JB: y = IB (IB - 1) / 2 + JB
    int IB = 1;
    while ((IB + 1) * IB / 2 <= y) ++IB;
    dw_block<T, TI, Q, P, false>(x, dt, cs_g, dy, dw, rm, H, G, K, hps, bkg, nbkg, slice, IB, y - IB * (IB - 1) / 2,
                             *reinterpret_cast<DwLds<T, P>*>(smem), dw_st);
  }
}

// ---------------------------------------------------------------------------
// The same head sums with a whole chunk per workgroup (bf16 storage, chunk
// 256, headdim 64).  Per ((b, k, g), head slice) two workgroups of 8 waves:
//   kind 0: the dC and dB partials of all Q rows (the sums of bc_heads_block)
//   kind 1: the lower triangle of dW (the sums of dw_block)
// The 64-row blocks of k_dw_heads read every head's dy and x rows and states
// once per block: about 352 KB of requests per head and item at dstate 128
// against 96 KB of distinct data.  Here each workgroup reads what it uses
// once (kind 0: dy, x, Hin, Gk; kind 1: dy, x), and the two workgroups of an
// item are dealt 8 dispatch slots apart, so they run on one XCD and the rows
// the second reads come from its L2.  The states (kind 0) and the x rows
// with the head's cs and dt (kind 1) travel global -> LDS by direct copies,
// one head ahead, into two buffers; each wave loads the row fragments of
// its own rows into registers one head ahead.  Kind 1 takes each head's
// 16x16 products of raw operands and applies the head's decay
// dt_j exp(cs_i - cs_j) and the causal mask to the product before adding
// it, so no operand is rescaled and rounded again.
template <typename TI, int N>
struct HsLayout {
  static constexpr int Q = 256, P = 64, NW = 8, NTH = NW * 64;
  static constexpr int SPC = P * N / 8;                  // 16-byte pieces of one state
  static constexpr int SPT = 2 * SPC / NTH;              // state copies per thread and head (Hin, Gk)
  static constexpr int XPR = P * (int)sizeof(TI) / 16;   // 16-byte pieces of an x row
  static constexpr int XPT = Q * XPR / NTH;              // x copies per thread and head
  static constexpr int XBYTES = Q * P * (int)sizeof(TI);
  static constexpr int BUF = (2 * P * N * 2 > XBYTES + 2 * Q * 4) ? 2 * P * N * 2 : XBYTES + 2 * Q * 4;
  static_assert(SPC % NTH == 0 && (Q * XPR) % NTH == 0, "whole copies per thread");
  static_assert(NTH % (N / 8) == 0 && (NTH / (N / 8)) % 16 == 0, "state copies keep the swizzle bits");
};

// State rows in LDS: row r's 32-byte segments (16 columns) are XOR-permuted
// by hs_key(r), so that the 16 rows one transposing read touches (rows
// 8q + t and 8q + 4 + t of a 32-row K step, t < 4) fall on distinct banks.
template <int N>
__device__ __forceinline__ int hs_key(int r) {
  return N >= 128 ? ((r & 3) | ((r >> 1) & 4)) : ((r & 3) ^ ((r >> 3) & 1));
}
// x rows in LDS: row r's 16-byte pieces are XOR-permuted by hs_xkey(r), so
// that the 16 rows a fragment read touches (a 16-aligned group) fall on
// distinct banks.  The key depends on r % 16 only, so a tile's rows share
// one per-lane offset.
template <typename TI>
__device__ __forceinline__ int hs_xkey(int r) {
  return sizeof(TI) == 2 ? ((r ^ ((r >> 3) & 1)) & 7) : ((r >> 2) & 3);
}

template <typename TI, int N>
__device__ __forceinline__ void hs_bc(const TI* __restrict__ x, const float* __restrict__ dt,
                                      const float* __restrict__ cs_g, const bf16* __restrict__ dy,
                                      const bf16* __restrict__ hin, const bf16* __restrict__ gst,
                                      float* __restrict__ dcpart, float* __restrict__ dbpart, const RowMap& rm,
                                      int H, int G, int K, int hps, int bkg, int nbkg, int slice, bf16* S0,
                                      bf16* S1) {
  typedef bf16 T;
  typedef HsLayout<TI, N> Ly;
  constexpr int Q = Ly::Q, P = Ly::P, NTH = Ly::NTH, SPT = Ly::SPT, SPC = Ly::SPC;
  constexpr int TN = N / 16, RPC = N / 8;
  constexpr bool F8 = std::is_same<TI, fp8>::value;
  typedef typename std::conditional<F8, uint2, bf16x8>::type XR;  // raw x piece of a fragment

  const int g = bkg % G, bk = bkg / G, k = bk % K, b = bk / K;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), l = lane_id(), q = l >> 4, c = l & 15;
  const int t = threadIdx.x;
  const int64_t row0 = chunk_row0(rm, b, k, Q);
  x = rows_in(rm, k, x, rm.x);
  dy = rows_in(rm, k, dy, rm.dy);
  const int hpg = H / G, h0 = g * hpg + slice * hps, nh = min(hps, hpg - slice * hps);

  // copy n of thread t fills LDS piece n NTH + t: state (n NTH) / SPC, row
  // ((n NTH) % SPC) / RPC + t / RPC; rows advance by multiples of 16 between
  // copies, which keeps the key
  const int sr = t / RPC, sp = t % RPC;
  const int so0 = sr * N + ((((sp >> 1) ^ hs_key<N>(sr)) << 1) | (sp & 1)) * 8;
  auto dma = [&](int hh, T* Sb) {
    const int64_t st = (((int64_t)b * K + k) * H + h0 + hh) * P * N;
#pragma unroll
    for (int n = 0; n < SPT; ++n) {
      const T* src = ((n * NTH) / SPC == 0 ? hin : gst) + st + ((n * NTH) % SPC) * 8 + so0;
      lds_copy16(src, Sb + (n * NTH + wave * kWave) * 8);
    }
  };
  struct Regs {
    bf16x8 ad[2][2];  // dy rows 32 wave + 16 tt + c, K = 32 kp + 8 q ..
    XR ax[2][2];      // x rows, the same pieces
    float cs[2], dt[2], cl;
  };
  const int ioff = (32 * wave + c) * H * P + 8 * q;  // this lane's first row, its K piece
  auto load_regs = [&](Regs& R, int hh) {
    const int h = h0 + hh;
    const T* dyh = dy + (row0 * H + h) * P + ioff;
    const TI* xh = x + (row0 * H + h) * P + ioff;
    const float* csb = cs_g + (((int64_t)b * H + h) * K + k) * Q;
    const float* dtb = dt + (((int64_t)b * H + h) * K + k) * Q;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        R.ad[tt][kp] = *reinterpret_cast<const bf16x8*>(dyh + 16 * tt * H * P + 32 * kp);
        R.ax[tt][kp] = *reinterpret_cast<const XR*>(xh + 16 * tt * H * P + 32 * kp);
      }
      R.cs[tt] = csb[32 * wave + 16 * tt + c];
      R.dt[tt] = dtb[32 * wave + 16 * tt + c];
    }
    R.cl = csb[Q - 1];
  };

  f4 accC[2][TN], accB[2][TN];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) accC[tt][tn] = accB[tt][tn] = f4{0.f, 0.f, 0.f, 0.f};
  // transposing reads: lane (q, c) addresses row 32 kp + 8 q + c / 4 (and 4
  // rows below), columns 16 tn + 4 (c % 4) .. of its segment
  const int kr = 8 * q + (c >> 2), key = hs_key<N>(kr);
  const int roff = kr * N + 4 * (c & 3);
  auto compute = [&](Regs& R, const T* Sb) {
    // the row fragments, scaled in place: dC rows by exp(cs_i), dB rows by
    // exp(cs_last - cs_j) dt_j
    Frag<T> fc[2][2], fb[2][2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const float sc = __expf(R.cs[tt]);
      const float sb = __expf(R.cl - R.cs[tt]) * R.dt[tt];
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        bf16x8 xr;
        if constexpr (F8) xr = e4m3x8_to_bf16(R.ax[tt][kp]);
        else xr = R.ax[tt][kp];
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
          R.ad[tt][kp][s8] = (bf16)((float)R.ad[tt][kp][s8] * sc);
          xr[s8] = (bf16)((float)xr[s8] * sb);
        }
        fc[tt][kp].v = R.ad[tt][kp];
        fb[tt][kp].v = xr;
      }
    }
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const T* a = Sb + 32 * kp * N + roff + ((tn ^ key) << 4);
        Frag<T> bh, bg;
        frag_load_kmajor_at(bh, a, a + 4 * N);
        frag_load_kmajor_at(bg, a + P * N, a + P * N + 4 * N);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          mma(accC[tt][tn], fc[tt][kp], bh);
          mma(accB[tt][tn], fb[tt][kp], bg);
        }
      }
    }
  };

  // Head hh lives in buffer hh & 1.  At the top of a head its copies and row
  // loads (issued one head earlier) are waited for; after the barrier the
  // other buffer is free (the previous head is done with it) and takes the
  // next head's copies.  Unrolled by two so that every LDS access names its
  // buffer's array.
  Regs R0, R1;
  dma(0, S0);
  load_regs(R0, 0);
  auto step = [&](int hh, Regs& Rc, Regs& Rn, const T* Sb, T* Sn) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (hh + 1 < nh) {
      dma(hh + 1, Sn);
      load_regs(Rn, hh + 1);
    }
    compute(Rc, Sb);
  };
  for (int hh = 0; hh < nh; hh += 2) {
    step(hh, R0, R1, S0, S1);
    if (hh + 1 < nh) step(hh + 1, R1, R0, S1, S0);
  }

  const int64_t prow0 = ((int64_t)b * K + k) * Q;
  float* oc = dcpart + (int64_t)slice * nbkg * Q * N;
  float* ob = dbpart + (int64_t)slice * nbkg * Q * N;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t o = ((prow0 + 32 * wave + 16 * tt + 4 * q + r) * G + g) * N + c;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        oc[o + 16 * tn] = accC[tt][tn][r];
        ob[o + 16 * tn] = accB[tt][tn][r];
      }
    }
}

template <typename TI, int N>
__device__ __forceinline__ void hs_dw(const TI* __restrict__ x, const float* __restrict__ dt,
                                      const float* __restrict__ cs_g, const bf16* __restrict__ dy,
                                      float* __restrict__ dw, const RowMap& rm, int H, int G, int K, int hps, int bkg,
                                      int nbkg, int slice, TI* X0, TI* X1, float* C0, float* C1, int dw_st) {
  typedef bf16 T;
  typedef HsLayout<TI, N> Ly;
  constexpr int Q = Ly::Q, P = Ly::P, NTH = Ly::NTH, XPR = Ly::XPR, XPT = Ly::XPT;
  constexpr int NT = Q / 16, EPP = 16 / (int)sizeof(TI);
  constexpr int NS = NT + 1;  // tiles per wave: row tiles NT - 1 - wave and wave
  constexpr bool F8 = std::is_same<TI, fp8>::value;
  static_assert(NT == 2 * Ly::NW, "two row tiles per wave");

  const int g = bkg % G, bk = bkg / G, k = bk % K, b = bk / K;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), l = lane_id(), q = l >> 4, c = l & 15;
  const int t = threadIdx.x;
  const int64_t row0 = chunk_row0(rm, b, k, Q);
  x = rows_in(rm, k, x, rm.x);
  dy = rows_in(rm, k, dy, rm.dy);
  const int hpg = H / G, h0 = g * hpg + slice * hps, nh = min(hps, hpg - slice * hps);
  // slot s < NT - wave: tile (ti1, s); else (ti0, NT - s).  The first NT / 2
  // slots always belong to ti1 (wave < NT / 2).
  const int ti1 = NT - 1 - wave, ti0 = wave;

  // copy n of thread t fills LDS piece n NTH + t: row n NTH / XPR + t / XPR
  // (the step keeps the key); the head's cs and dt come with waves 0 and 1
  const int xr0 = t / XPR;
  const int xo0 = xr0 * H * P + ((t % XPR) ^ hs_xkey<TI>(xr0)) * EPP;
  auto dma = [&](int hh, TI* Xb, float* Cb) {
    const int h = h0 + hh;
    const TI* xh = x + (row0 * H + h) * P + xo0;
#pragma unroll
    for (int n = 0; n < XPT; ++n) lds_copy16(xh + n * (NTH / XPR) * H * P, Xb + (n * NTH + wave * kWave) * EPP);
    if (wave < 2) {
      const float* src = (wave == 0 ? cs_g : dt) + (((int64_t)b * H + h) * K + k) * Q + 4 * l;
      lds_copy16(src, Cb + wave * kWave * 4);
    }
  };
  struct Regs {
    bf16x8 ad[2][2];  // dy rows 16 ti + c of the row tiles (ti0, ti1), K = 32 kp + 8 q ..
  };
  auto load_regs = [&](Regs& R, int hh) {
    const T* dyh = dy + (row0 * H + h0 + hh) * P + c * H * P + 8 * q;
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      R.ad[0][kp] = *reinterpret_cast<const bf16x8*>(dyh + 16 * ti0 * H * P + 32 * kp);
      R.ad[1][kp] = *reinterpret_cast<const bf16x8*>(dyh + 16 * ti1 * H * P + 32 * kp);
    }
  };
  auto slot = [&](int s, int& ti, int& tj) {
    const bool first = s < NT / 2 || s < NT - wave;
    ti = first ? ti1 : ti0;
    tj = first ? s : NT - s;
    return first;
  };

  f4 acc[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) acc[s] = f4{0.f, 0.f, 0.f, 0.f};
  // per-lane parts of the fragment reads of x row 16 tj + c (K = 32 kp + 8 q ..)
  int xl[2];
#pragma unroll
  for (int kp = 0; kp < 2; ++kp)
    xl[kp] = F8 ? c * P + ((2 * kp + (q >> 1)) ^ hs_xkey<TI>(c)) * EPP + 8 * (q & 1)
                : c * P + ((4 * kp + q) ^ hs_xkey<TI>(c)) * EPP;
  auto compute = [&](const Regs& R, const TI* Xb, const float* Cb) {
    // The per-lane offsets pass through an empty asm at every head, so the
    // 17 slots' addresses and masks are formed here instead of being hoisted
    // out of the head loop (where they took more registers than there are).
    int xo[2] = {xl[0], xl[1]}, cl = c, mb = 4 * q - c;
    asm volatile("" : "+v"(xo[0]), "+v"(xo[1]), "+v"(cl), "+v"(mb));
    const f4 cs0 = *reinterpret_cast<const f4*>(&Cb[16 * ti0 + 4 * q]);
    const f4 cs1 = *reinterpret_cast<const f4*>(&Cb[16 * ti1 + 4 * q]);
    // Below the diagonal tile (every i after every j) the decay splits at the
    // row tile's first token r: exp(cs_i - cs_r) exp(cs_r - cs_j), both
    // factors <= 1, so a lane forms its 4 row factors per row tile once per
    // head and one column factor per tile instead of 4 exponentials per tile.
    const float cr0 = Cb[16 * ti0], cr1 = Cb[16 * ti1];
    f4 rf0, rf1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      rf0[r] = __expf(cs0[r] - cr0);
      rf1[r] = __expf(cs1[r] - cr1);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      int ti, tj;
      const bool first = slot(s, ti, tj);
      const TI* xt = Xb + 16 * tj * P;
      Frag<T> fb[2];
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        if constexpr (F8) fb[kp].v = e4m3x8_to_bf16(*reinterpret_cast<const uint2*>(xt + xo[kp]));
        else fb[kp].v = *reinterpret_cast<const bf16x8*>(xt + xo[kp]);
      }
      f4 dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        Frag<T> fa;
        fa.v = first ? R.ad[1][kp] : R.ad[0][kp];
        mma(dp, fa, fb[kp]);
      }
      const float csj = Cb[16 * tj + cl], dtj = Cb[Q + 16 * tj + cl];
      if (ti != tj) {  // wave-uniform
        const f4 rf = first ? rf1 : rf0;
        const float cf = dtj * __expf((first ? cr1 : cr0) - csj);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[s][r] += dp[r] * (rf[r] * cf);
      } else {  // the diagonal tile: masked, one exponential per element
        const f4 csi = first ? cs1 : cs0;
        const int d = mb;  // row i - column j = d + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = dp[r] * (dtj * __expf(csi[r] - csj));
          acc[s][r] += (d + r >= 0) ? v : 0.0f;
        }
      }
    }
  };

  Regs R0, R1;
  dma(0, X0, C0);
  load_regs(R0, 0);
  auto step = [&](int hh, const Regs& Rc, Regs& Rn, const TI* Xb, const float* Cb, TI* Xn, float* Cn) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (hh + 1 < nh) {
      dma(hh + 1, Xn, Cn);
      load_regs(Rn, hh + 1);
    }
    compute(Rc, Xb, Cb);
  };
  for (int hh = 0; hh < nh; hh += 2) {
    step(hh, R0, R1, X0, C0, X1, C1);
    if (hh + 1 < nh) step(hh + 1, R1, R0, X1, C1, X0, C0);
  }

  // the tiles, then zeros above the diagonal inside the 64-row diagonal
  // blocks (the dC / dB finalisation reads whole 64 x 64 blocks)
  auto store = [&](auto* o) {  // o: this item's Q x Q dW
    typedef typename std::remove_pointer<decltype(o)>::type O;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      int ti, tj;
      slot(s, ti, tj);
      O* p = o + (16 * ti + 4 * q) * Q + 16 * tj + c;
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r * Q] = from_f<O>(acc[s][r]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ti = u ? ti1 : ti0;
      O* p = o + (16 * ti + 4 * q) * Q + c;
      for (int tj = ti + 1; tj <= (ti | 3); ++tj)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r * Q + 16 * tj] = from_f<O>(0.0f);
    }
  };
  if (dw_st) store(reinterpret_cast<T*>(dw) + (int64_t)bkg * Q * Q);
  else store(dw + ((int64_t)slice * nbkg + bkg) * Q * Q);
}

template <typename TI, int N>
__global__ __launch_bounds__(512, 1) void k_head_sums(const TI* __restrict__ x, const float* __restrict__ dt,
                                                      const float* __restrict__ cs_g, const bf16* __restrict__ dy,
                                                      const bf16* __restrict__ hin, const bf16* __restrict__ gst,
                                                      float* __restrict__ dw, float* __restrict__ dcpart,
                                                      float* __restrict__ dbpart, const RowMap rm, int H, int G,
                                                      int K, int hps, int nbkg, int nitems, int dw_st) {
  typedef HsLayout<TI, N> Ly;
  // two head buffers, each its own array (see the head loops)
  __shared__ __attribute__((aligned(16))) unsigned char B0[Ly::BUF], B1[Ly::BUF];
  const int xcd = blockIdx.x % 8, j = blockIdx.x / 8;
  const int item = (j >> 1) * 8 + xcd;
  if (item >= nitems) return;  // whole workgroup, before any barrier
  const int bkg = item % nbkg, slice = item / nbkg;
  if ((j & 1) == 0)
    hs_bc<TI, N>(x, dt, cs_g, dy, hin, gst, dcpart, dbpart, rm, H, G, K, hps, bkg, nbkg, slice,
                 reinterpret_cast<bf16*>(B0), reinterpret_cast<bf16*>(B1));
  else
    hs_dw<TI, N>(x, dt, cs_g, dy, dw, rm, H, G, K, hps, bkg, nbkg, slice, reinterpret_cast<TI*>(B0),
                 reinterpret_cast<TI*>(B1), reinterpret_cast<float*>(B0 + Ly::XBYTES),
                 reinterpret_cast<float*>(B1 + Ly::XBYTES), dw_st);
}

// ---------------------------------------------------------------------------
// dC / dB for one (b, k, g) and one 64-row block RB: the head-slice partials
// summed in slice order, plus the dW part
//   dC_i = ... + sum_{j <= i} dW_ij B_j        dB_j = ... + sum_{i >= j} dW_ij C_i
// with dW the fixed-order sum of its head-slice partials.  K = tokens, in
// 64-token blocks: the dW block (converted to the storage type) and the B
// (or C) rows are staged row-major in LDS; dC reads dW rows directly, dB reads
// them K-major, and B / C are read K-major (transposing LDS read).
// A block takes one of NH parts of the dstate columns (more workgroups for a
// launch that has only b K G (Q / 64) row blocks); each part stages its own
// B / C columns and the whole dW block.
template <typename T, int Q, int N, int NH>
struct BcFinalLds {
  static constexpr int NP = N / NH;
  static constexpr int WP = 64 + 16;         // row pitches (8 mod 16 dwords)
  static constexpr int MP = NP + ((24 - (NP * (int)sizeof(T) / 4) % 16) % 16) * 4 / (int)sizeof(T);
  __attribute__((aligned(16))) T Wb[64][WP];
  __attribute__((aligned(16))) T Ms[64][MP];
};

template <typename T, typename TI, int Q, int N, bool DB, int NH, bool DWST>
__device__ __forceinline__ void bc_final_block(const float* __restrict__ part, const float* __restrict__ dw,
                                               const TI* __restrict__ M, T* __restrict__ out, const RowMap& rm,
                                               int G, int K, int nslice, int nslice_dw, int bkg, int nbkg, int RB,
                                               int zpart, BcFinalLds<T, Q, N, NH>& sm) {
  constexpr int NTH = 256;
  constexpr int NP = N / NH;                 // dstate columns of this part
  constexpr int TN = NP / 16, NB = Q / 64;
  constexpr int VN = Vec16<T>::n;
  constexpr int WP = BcFinalLds<T, Q, N, NH>::WP, MP = BcFinalLds<T, Q, N, NH>::MP;
  constexpr int MPIECES = 64 * NP / VN;
  constexpr int MPT = (MPIECES + NTH - 1) / NTH;
  static_assert(N % NH == 0 && NP % 16 == 0, "dstate parts");
  typedef typename Vec16<T>::type V;
  auto& Wb = sm.Wb;
  auto& Ms = sm.Ms;

  const int n0 = NP * zpart;
  const int g = bkg % G, bk = bkg / G, k = bk % K, b = bk / K;
  const int wave = threadIdx.x / kWave, l = lane_id(), q = l >> 4, c = l & 15;
  const int64_t row0 = chunk_row0(rm, b, k, Q);
  M = rows_in(rm, k, M, DB ? rm.C : rm.B);
  out = rows_out(rm, k, out, DB ? rm.dB : rm.dC);
  const int64_t prow0 = ((int64_t)b * K + k) * Q;  // row of the fp32 partials (chunk rows)
  const int r0 = 64 * RB;
  const int64_t dws = (int64_t)nbkg * Q * Q;  // dW slice stride
  const float* dwb = dw + (int64_t)bkg * Q * Q;

  f4 acc[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) acc[tn] = f4{0.f, 0.f, 0.f, 0.f};

  // The operands of one block kb in registers: the dW block's 4-element runs
  // and the M rows.  With dW in the storage type (DWST: a single head slice,
  // the case of problems with many (b, k, g) items) block kb + 1 is loaded
  // while block kb's products run; the fp32 head-slice partials (several
  // slices: problems with few items, where the registers the prefetch takes
  // cost more occupancy than it gains) are loaded, added and staged in turn.
  constexpr int WRUNS = 64 * 64 / 4 / NTH;  // 4-element dW runs per thread
  static_assert(64 * 64 % (4 * NTH) == 0, "dW runs");
  typedef typename Vec4<T>::type W4;
  [[maybe_unused]] W4 wst[WRUNS];
  [[maybe_unused]] f4 wsl[WRUNS];
  V mv[MPT];
  const int kb0 = DB ? RB : 0, kb1 = DB ? NB - 1 : RB;
  auto load_block = [&](int kb) {
    const int ib = DB ? kb : RB, jb = DB ? RB : kb;  // dW rows i, columns j
    auto eo_of = [&](int it) {
      const int e = (threadIdx.x + NTH * it) * 4, il = e / 64, jl = e % 64;
      return (int64_t)(64 * ib + il) * Q + 64 * jb + jl;
    };
    if constexpr (DWST) {  // one slice, already in the storage dtype
#pragma unroll
      for (int it = 0; it < WRUNS; ++it)
        wst[it] = *reinterpret_cast<const W4*>(reinterpret_cast<const T*>(dw) + (int64_t)bkg * Q * Q + eo_of(it));
    } else {
      // slice by slice, each slice's loads issued together (the sum per
      // element runs over the slices in order either way)
#pragma unroll
      for (int it = 0; it < WRUNS; ++it) wsl[it] = *reinterpret_cast<const f4*>(dwb + eo_of(it));
      for (int z = 1; z < nslice_dw; ++z)
#pragma unroll
        for (int it = 0; it < WRUNS; ++it) wsl[it] += *reinterpret_cast<const f4*>(dwb + eo_of(it) + z * dws);
    }
    // B rows j (dC) or C rows i (dB) of block kb
#pragma unroll
    for (int n = 0; n < MPT; ++n) {
      const int u = threadIdx.x + NTH * n;
      if (MPIECES % NTH == 0 || u < MPIECES) {
        const int rr = u / (NP / VN), cu = u % (NP / VN);
        mv[n] = load_vec16<T, TI>(M + ((row0 + 64 * kb + rr) * G + g) * N + n0 + cu * VN);
      }
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int it = 0; it < WRUNS; ++it) {
      const int e = (threadIdx.x + NTH * it) * 4, il = e / 64, jl = e % 64;
      W4 w;
      if constexpr (DWST) {
        w = wst[it];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = from_f<T>(wsl[it][r]);
      }
      *reinterpret_cast<W4*>(&Wb[il][jl]) = w;
    }
#pragma unroll
    for (int n = 0; n < MPT; ++n) {
      const int u = threadIdx.x + NTH * n;
      if (MPIECES % NTH == 0 || u < MPIECES) {
        const int rr = u / (NP / VN), cu = u % (NP / VN);
        *reinterpret_cast<V*>(&Ms[rr][cu * VN]) = mv[n];
      }
    }
  };
  const int64_t ps = (int64_t)nbkg * Q * N;  // head-slice partial stride b*K*G*Q*N
  auto pidx = [&](int tn, int r) {
    return ((prow0 + r0 + 16 * wave + 4 * q + r) * G + g) * N + n0 + 16 * tn + c;
  };
  if constexpr (DWST) load_block(kb0);
  for (int kb = kb0; kb <= kb1; ++kb) {
    if (kb > kb0) __syncthreads();  // the previous block is no longer read
    if constexpr (!DWST) load_block(kb);
    store_block();
    __syncthreads();
    if constexpr (DWST) {
      if (kb < kb1) load_block(kb + 1);
    }
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      Frag<T> fa;
      if (DB) frag_load_kmajor<64>(fa, &Wb[0][0], WP, kp * 32, 16 * wave, q, c);   // row j, K = i
      else frag_load2(fa, &Wb[16 * wave + c][kp * 32 + 4 * q], &Wb[16 * wave + c][kp * 32 + 16 + 4 * q]);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        Frag<T> fb;
        frag_load_kmajor<64>(fb, &Ms[0][0], MP, kp * 32, 16 * tn, q, c);
        mma(acc[tn], fa, fb);
      }
    }
  }
  // the head-slice partials slice by slice, each slice's loads issued together
  float pv[TN][4];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int r = 0; r < 4; ++r) pv[tn][r] = part[pidx(tn, r)];
  for (int z = 1; z < nslice; ++z)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[tn][r] += part[z * ps + pidx(tn, r)];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      out[((row0 + r0 + 16 * wave + 4 * q + r) * G + g) * N + n0 + 16 * tn + c] = from_f<T>(pv[tn][r] + acc[tn][r]);
  }
}

// dC and dB in one launch (both read the same dW blocks).  With one dstate
// part (many (b, k, g) items), each item's 2 Q/64 workgroups (row block, dC
// or dB) are dealt 8 dispatch slots apart, so that they run on one XCD at
// about the same time and the item's dW blocks and B / C rows, which several
// of them read, come from that XCD's L2 after the first (the blocks with the
// most 64-token steps first): at the long context this took the launch from
// 1.81 GB of HBM traffic toward its 1.24 GB of distinct data.  With several
// dstate parts (few items) the grid is (item, row block, part and kind),
// which measured faster there.
template <typename T, typename TI, int Q, int N, int NH, bool DWST>
__global__ __launch_bounds__(256) void k_bc_final(const float* __restrict__ dcpart, const float* __restrict__ dbpart,
                                                  const float* __restrict__ dw, const TI* __restrict__ B,
                                                  const TI* __restrict__ C, T* __restrict__ dC, T* __restrict__ dB,
                                                  const RowMap rm, int G, int K, int nslice, int nbkg) {
  constexpr int NB = Q / 64;
  __shared__ BcFinalLds<T, Q, N, NH> sm;
  if constexpr (NH == 1) {
    const int xcd = blockIdx.x % 8, j = blockIdx.x / 8;
    const int blk = j % (2 * NB), item = (j / (2 * NB)) * 8 + xcd;
    if (item >= nbkg) return;  // whole workgroup, before any barrier
    const int steps = NB - blk / 2;  // 64-token steps of this block, NB down to 1
    if (blk & 1)
      bc_final_block<T, TI, Q, N, true, NH, DWST>(dbpart, dw, C, dB, rm, G, K, nslice, nslice, item, nbkg, NB - steps,
                                                  0, sm);
    else
      bc_final_block<T, TI, Q, N, false, NH, DWST>(dcpart, dw, B, dC, rm, G, K, nslice, nslice, item, nbkg, steps - 1,
                                                   0, sm);
  } else {  // blockIdx.z < NH: dstate part z of dC; the rest: the parts of dB
    const int z = blockIdx.z;
    if (z < NH)
      bc_final_block<T, TI, Q, N, false, NH, DWST>(dcpart, dw, B, dC, rm, G, K, nslice, nslice, blockIdx.x, gridDim.x,
                                                   blockIdx.y, z, sm);
    else
      bc_final_block<T, TI, Q, N, true, NH, DWST>(dbpart, dw, C, dB, rm, G, K, nslice, nslice, blockIdx.x, gridDim.x,
                                                  blockIdx.y, z - NH, sm);
  }
}

// Fixed-order sums of the per-(b, k) partials (dA, dD and, when requested,
// the dt bias gradient): one workgroup per head; each thread sums a strided
// slice, then a fixed tree combines the slices.
__global__ __launch_bounds__(256) void k_da_dd(const float* __restrict__ dapart, const float* __restrict__ ddpart,
                                               const float* __restrict__ dbiaspart, float* __restrict__ dA,
                                               float* __restrict__ dD, float* __restrict__ dbias, int BK, int H) {
  __shared__ float ra[4], rd[4], rb[4];
  const int h = blockIdx.x;
  float sa = 0.0f, sd = 0.0f, sb = 0.0f;
  for (int i = threadIdx.x; i < BK; i += 256) {
    sa += dapart[(int64_t)i * H + h];
    sd += ddpart[(int64_t)i * H + h];
    if (dbias) sb += dbiaspart[(int64_t)i * H + h];
  }
  sa = wave_sum(sa);
  sd = wave_sum(sd);
  if (dbias) sb = wave_sum(sb);
  const int wave = threadIdx.x / kWave;
  if (lane_id() == 0) { ra[wave] = sa; rd[wave] = sd; rb[wave] = sb; }
  __syncthreads();
  if (threadIdx.x == 0) {
    dA[h] = (ra[0] + ra[1]) + (ra[2] + ra[3]);
    dD[h] = (rd[0] + rd[1]) + (rd[2] + rd[3]);
    if (dbias) dbias[h] = (rb[0] + rb[1]) + (rb[2] + rb[3]);
  }
}

// dstate parts of k_bc_final: 32 columns each
template <int N> constexpr int kBcParts = N >= 32 ? N / 32 : 1;

template <typename T, typename TI, int Q, int P, int N>
void run_bwd(const Layout& lay, const BwdArgs& a, hipStream_t st, const ssd_probe* probe) {
  const int b = (int)lay.b, H = (int)lay.H, G = (int)lay.G, K = (int)lay.K;
  const TI* x = static_cast<const TI*>(a.x);
  const float* dt = a.dtf;  // the step, float32, as the forward's cumsum wrote it
  const TI* B = static_cast<const TI*>(a.B);
  const TI* C = static_cast<const TI*>(a.C);
  const T* dy = static_cast<const T*>(a.dy);
  const T* hin = static_cast<const T*>(a.hin);
  T* gst = static_cast<T*>(a.gst);
  {
    ProbeScope ps(probe, SSD_K_CHUNK_STATE_BWD, st);
    launch_chunk_state<T, T, TI, Q, P, N, true>(dy, C, dt, a.cs, static_cast<T*>(a.dhloc), hin, a.dlpart, a.rows, b, H,
                                                G, K, st);
  }
  {
    ProbeScope ps(probe, SSD_K_STATE_PASSING_BWD, st);
    const int PN = P * N;
    k_state_passing<T, Q, true><<<dim3((PN / 4 + 255) / 256, b * H), dim3(256), 0, st>>>(static_cast<const T*>(a.dhloc), a.cs, a.dfinal, gst, a.dinit, H, K, PN);
  }
  {
    ProbeScope ps(probe, SSD_K_CHUNK_SCAN_BWD, st);
    // resident over heads where a slice holds enough heads (resident_slices);
    // it writes the row sums of every split into the first split's row
    // measured with k_dl_assemble, 20 heads (2.7B shape) 0.352 -> 0.276 ms,
    // 14 (Zamba2-7B-like) 0.222 -> 0.178 ms, 10 (long context) 1.34 -> 1.15 ms,
    // 8 (Mamba2-370M shape) 0.154 -> 0.122 ms
    int RS = 1;
    const int rper = resident_slices(b * K * G, H / G, &RS);
    const bool res_bwd = std::is_same<T, bf16>::value && Q == 256 && P == 64 && N % 64 == 0 && rper >= kMinResidentHeadsBwd;
    if constexpr (std::is_same<T, bf16>::value && Q == 256 && P == 64 && N % 64 == 0) {
      if (res_bwd) {
        const int nbkg = b * K * G;
        k_chunk_scan_bwd_heads<TI, N><<<dim3((nbkg + 7) / 8 * 8 * RS), dim3(512), 0, st>>>(
            x, dt, a.cs, a.D, B, C, hin, gst, dy, static_cast<T*>(a.dx), a.dlpart, a.dlscal, a.rows, H, G, K, rper, RS,
            nbkg);
      }
    }
    if (!res_bwd) {
      const int nitems = b * K * H;
      k_chunk_scan_bwd<T, TI, Q, P, N><<<dim3(xcd_grid(nitems) * scan_bwd_splits(Q)), dim3(256), 0, st>>>(
          x, dt, a.cs, a.D, B, C, hin, gst, dy, static_cast<T*>(a.dx), a.dlpart, a.dlscal, nitems, a.rows, H, G, K);
    }
    const dim3 dlg((b * K + 7) / 8 * 8 * ((H + 3) / 4));
    if (res_bwd)
      k_dl_assemble<T, Q, 1, 1><<<dlg, dim3(256), 0, st>>>(
          a.dlpart, a.dlscal, a.cs, dt, a.A, static_cast<T*>(a.ddt), a.dapart, a.ddpart, a.dbiaspart, a.rows, H, K,
          a.softplus, b * K);
    else
      k_dl_assemble<T, Q, 1, scan_bwd_splits(Q)><<<dlg, dim3(256), 0, st>>>(
          a.dlpart, a.dlscal, a.cs, dt, a.A, static_cast<T*>(a.ddt), a.dapart, a.ddpart, a.dbiaspart, a.rows, H, K,
          a.softplus, b * K);
  }
  const int hpg = H / G, S = (int)lay.nslice, hps = (hpg + S - 1) / S;
  const int nbkg = b * K * G;
  // one head slice: dW goes straight to the storage dtype (bit-identical, as the
  // dC/dB products round it to that type anyway) at half the bytes
  const int dw_st = (S == 1 && sizeof(T) == 2) ? 1 : 0;
  {
    ProbeScope ps(probe, SSD_K_DW_HEADS, st);
    const int nb = Q / 64, nitems = nbkg * S;
    if constexpr (std::is_same<T, bf16>::value && Q == 256 && P == 64 && N % 64 == 0) {
      k_head_sums<TI, N><<<dim3((nitems + 7) / 8 * 8 * 2), dim3(HsLayout<TI, N>::NTH), 0, st>>>(
          x, dt, a.cs, dy, hin, gst, a.dw, a.dcpart, a.dbpart, a.rows, H, G, K, hps, nbkg, nitems, dw_st);
    } else {
      k_dw_heads<T, TI, Q, P, N><<<dim3((nitems + 7) / 8 * 8 * (2 * nb + nb * (nb + 1) / 2)), dim3(256), 0, st>>>(
          x, dt, a.cs, dy, hin, gst, a.dw, a.dcpart, a.dbpart, a.rows, H, G, K, hps, nbkg, nitems, dw_st);
    }
  }
  {
    ProbeScope ps(probe, SSD_K_BC_FINAL, st);
    // Splitting the dstate columns gives a launch with few (b, k, g) items enough
    // workgroups, but every part stages and converts the whole dW block again;
    // once the row blocks alone make 2048 workgroups, one part takes all columns.
    auto launch = [&](auto nh, auto dwst) {
      constexpr int NH = decltype(nh)::value;
      const dim3 grid = NH == 1 ? dim3((nbkg + 7) / 8 * 8 * 2 * (Q / 64)) : dim3(nbkg, Q / 64, 2 * NH);
      k_bc_final<T, TI, Q, N, NH, decltype(dwst)::value><<<grid, dim3(256), 0, st>>>(
          a.dcpart, a.dbpart, a.dw, B, C, static_cast<T*>(a.dC), static_cast<T*>(a.dB), a.rows, G, K, S, nbkg);
    };
    using one = std::integral_constant<int, 1>;
    using parts = std::integral_constant<int, kBcParts<N>>;
    using st1 = std::integral_constant<bool, sizeof(T) == 2>;  // dw_st: dW in the storage type
    if ((int64_t)nbkg * (Q / 64) * 2 >= 2048) {
      if (dw_st) launch(one{}, st1{});
      else launch(one{}, std::false_type{});
    } else {
      if (dw_st) launch(parts{}, st1{});
      else launch(parts{}, std::false_type{});
    }
  }
  {
    ProbeScope ps(probe, SSD_K_DA_DD, st);
    k_da_dd<<<dim3(H), dim3(256), 0, st>>>(a.dapart, a.ddpart, a.dbiaspart, a.dA, a.dD,
                                           a.softplus ? a.ddt_bias : nullptr, b * K, H);
  }
}

#define SSD_INST_BWD_BF16(Q_, P_, N_) template void run_bwd<bf16, bf16, Q_, P_, N_>(const Layout&, const BwdArgs&, hipStream_t, const ssd_probe*);
#define SSD_INST_BWD_FP8(Q_, P_, N_) template void run_bwd<bf16, fp8, Q_, P_, N_>(const Layout&, const BwdArgs&, hipStream_t, const ssd_probe*);
#define SSD_INST_BWD_F32(Q_, P_, N_) template void run_bwd<float, float, Q_, P_, N_>(const Layout&, const BwdArgs&, hipStream_t, const ssd_probe*);
SSD_BF16_CONFIGS(SSD_INST_BWD_BF16)
SSD_BF16_CONFIGS(SSD_INST_BWD_FP8)
SSD_F32_CONFIGS(SSD_INST_BWD_F32)

}  // namespace ssd
