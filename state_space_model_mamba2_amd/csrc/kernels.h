// Internal launcher interface between the C-ABI layer (api.cpp) and the HIP
// kernels.  Not part of the public header.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ssd.h"

namespace ssd {

typedef __bf16 bf16;
typedef unsigned char fp8;  // OCP FP8 E4M3 code

// Workspace regions, all offsets in bytes from the workspace base and 256-byte aligned.
struct Layout {
  int64_t b, L, H, P, N, G, Q, K;
  size_t esz;  // bytes per storage element (2 for bf16, 4 for fp32)
  // saved workspace
  size_t cs_off, hin_off, wt_off, saved_bytes;
  // forward scratch
  size_t s_off, fwd_bytes;
  // backward scratch
  size_t dhloc_off, g_off, dw_off, dcpart_off, dbpart_off, dapart_off, ddpart_off, dlpart_off, dlscal_off,
      bwd_bytes;
  int64_t nslice;     // head slices of the dW / dC / dB head sums
  int64_t wtiles;  // 16x16 lower-triangle tiles per (batch, chunk, group)
};

// Token rows of the chunks.  Chunk k of sequence b starts at row b * L + k * Q
// of the caller's tensors.  When the sequence length is not a multiple of Q,
// the last chunk (k == kf) reads and writes zero-padded one-chunk copies
// instead ([b][Q] rows, sequence b's starting at row b * Q), so that every
// chunk has Q rows; kf = K when every chunk is whole.
struct RowMap {
  int64_t L;
  int kf;
  int lr;  // rows of chunk kf that hold tokens (L - kf * Q)
  const void *x, *dt, *B, *C, *dy;  // zero-padded inputs of chunk kf
  void *y, *dx, *ddt, *dB, *dC;     // its outputs, copied back afterwards
};

struct FwdArgs {
  const void *x, *dt, *B, *C;
  const float *A, *D;
  const float* init;  // [b][H][P][N] initial state, or null for zero
  int softplus;         // dt is the raw step: the scan uses softplus(dt + dt_bias)
  const float* dt_bias; // [H] or null (zero); read when softplus is set
  float* dtf;           // [b][H][K][Q] float32 step the scan uses, written by the cumsum (saved)
  void* y;
  float* final_state;
  RowMap rows;
  float* cs;    // [b][H][K][Q]
  void* hin;    // [b][K][H][P][N]  storage dtype
  void* S;      // [b][K][H][P][N], storage dtype
  void* wt;     // C.B^T tiles, forward lane order (forward scratch)
};

struct BwdArgs {
  const void *x, *dt, *B, *C, *dy;
  const float *A, *D;
  const float* cs;
  const void* hin;
  void *dx, *ddt, *dB, *dC;
  float *dA, *dD;
  const float* dfinal;  // [b][H][P][N] final-state cotangent, or null for zero
  const float* dtf;     // [b][H][K][Q] float32 step the forward used
  int softplus;         // dt was the raw step: ddt is chained through softplus
  float* ddt_bias;      // [H] gradient of dt_bias, or null
  float* dbiaspart;     // [b][K][H] per-chunk partials of ddt_bias (softplus only)
  float* dinit;         // [b][H][P][N] initial-state gradient, or null
  void* dhloc;     // [b][K][H][P][N], storage dtype
  void* gst;       // [b][K][H][P][N]  storage dtype: dL/d(state leaving chunk k)
  float* dw;       // [nslice][b][K][G][Q][Q], per-slice partials
  float* dcpart;   // [nslice][b][K][Q][G][N] fp32 partials of dC (chunk rows)
  float* dbpart;   // [nslice][b][K][Q][G][N] fp32 partials of dB (chunk rows)
  float* dapart;   // [b][K][H]
  float* ddpart;   // [b][K][H]
  float* dlpart;   // [b][K][H][dl_rows(Q)][Q]: per-token partial sums for dl
  float* dlscal;   // [b][K][H][scan_bwd_splits(Q) + 1]: <Gk, Hin_k> and per-split sum <dy, x>
  RowMap rows;
};

// Most head slices the group-level head sums of the backward split a group's
// heads into (each slice writes fp32 partials that are added in a fixed order).
constexpr int kMaxHeadSlices = 4;

// Workgroups that share one (batch, chunk, head) in the backward chunk kernel
// (each owns an interleaved half of the chunk's 16-token column tiles).
constexpr int scan_bwd_splits(int Q) { return Q >= 256 ? Q / 128 : 1; }
// Rows of per-token partial sums that dl is formed from, per (b, k, h): the
// splits' row sums of R, the column sums, q_j, <dxt_j, x_j> (chunk-scan
// gradient) and up to four headdim tiles' shares of the state-to-output term
// (chunk-state gradient).
constexpr int dl_rows(int Q) { return scan_bwd_splits(Q) + 7; }

// Kernel timing hook (see ssd_probe in the public header).
struct ProbeScope {
  const ssd_probe* p;
  int id;
  hipStream_t s;
  ProbeScope(const ssd_probe* p_, int id_, hipStream_t s_) : p(p_), id(id_), s(s_) {
    if (p && p->kernel == id) (void)hipEventRecord(p->start, s);
  }
  ~ProbeScope() {
    if (p && p->kernel == id) (void)hipEventRecord(p->stop, s);
  }
};

// Copies between the rows [row0, row0 + nvalid) of each of the b sequences
// of up to four tensors with row stride L and zero-padded [b][Q] row buffers
// (pad: the buffers' rows past nvalid get zero bytes; unpad: the nvalid rows
// are copied back), in one launch.  Row sizes are even; every pointer is
// 16-byte aligned.
struct RowCopy {
  const void* src[4];
  void* dst[4];
  int64_t rowbytes[4];
  int n;
};
void pad_rows(const RowCopy& c, int64_t L, int64_t row0, int64_t nvalid, int64_t Q, int64_t b, hipStream_t st);
void unpad_rows(const RowCopy& c, int64_t L, int64_t row0, int64_t nvalid, int64_t Q, int64_t b, hipStream_t st);

// Causal depthwise conv1d (conv.hip).
struct ConvArgs {
  int64_t b, L, C;
  int W, esz, silu;
  const void* x;        // [b][L][C]
  const float* w;       // [C][W]
  const float* bias;    // [C] or null
  const void* x_prev;   // [b][W-1][C] or null (zeros)
  void* y;              // forward output
  const void* dy;       // backward input
  void *dx, *dx_prev;   // backward outputs (dx_prev may be null)
  float *dw, *dbias;    // backward outputs (dbias may be null)
  float* part;          // [conv_partial_rows][C][W + 1] scratch
};
int64_t conv_partial_rows(int64_t b, int64_t L, int esz);
void run_conv_fwd(const ConvArgs& a, hipStream_t st);
void run_conv_bwd(const ConvArgs& a, hipStream_t st);

// T: compute and storage type of dt, y, states and tiles; TI: storage type of
// x, B and C (T, or fp8 with T = bf16).
template <typename T, typename TI, int Q, int P, int N>
void run_fwd(const Layout& lay, const FwdArgs& a, hipStream_t stream, const ssd_probe* probe);
template <typename T, typename TI, int Q, int P, int N>
void run_bwd(const Layout& lay, const BwdArgs& a, hipStream_t stream, const ssd_probe* probe);

}  // namespace ssd

// Compiled (chunk, headdim, dstate) combinations, per storage dtype.  The
// fp32 list is shorter because the backward chunk kernel's LDS staging of
// fp32 tiles must fit in 160 KiB per workgroup.  bf16 at chunk 64 is switched
// off: a GPU memory fault in that case under an earlier backward kernel was
// never traced to a cause, so the case stays unavailable until one is shown.
#define SSD_BF16_CONFIGS(X) \
  X(128, 16, 16) X(256, 16, 16) \
  X(128, 64, 64) X(256, 64, 64) \
  X(128, 64, 128) X(256, 64, 128)
#define SSD_F32_CONFIGS(X) \
  X(64, 16, 16) X(128, 16, 16) X(256, 16, 16) \
  X(64, 64, 64) X(128, 64, 64) \
  X(64, 64, 128)
