// C-ABI entry points of libssd: argument checks, workspace layout and
// dispatch to the compiled (dtype, chunk, headdim, dstate) instantiations.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "kernels.h"

// Forward scratch of ssd_fwd_noalloc: a device global, so every GPU the
// library runs on holds its own copy (allocated when the code object is
// loaded on that GPU, kept until the process ends).  Host code never uses
// this name as an address: the device address of each GPU's copy comes from
// hipGetSymbolAddress (static_scratch below).
static __device__ __align__(256) unsigned char scratch[SSD_FWD_STATIC_SCRATCH_BYTES];

namespace ssd {
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool is_supported(int dtype, int64_t Q, int64_t P, int64_t N) {
#define SSD_MATCH(Q_, P_, N_) if (Q == Q_ && P == P_ && N == N_) return true;
  if (dtype == SSD_BF16 || dtype == SSD_FP8) { SSD_BF16_CONFIGS(SSD_MATCH) }
  if (dtype == SSD_F32) { SSD_F32_CONFIGS(SSD_MATCH) }
#undef SSD_MATCH
  return false;
}

ssd_status check_shape(const ssd_shape* s) {
  if (!s) return SSD_ERR_INVALID_ARGUMENT;
  if (s->batch <= 0 || s->seqlen <= 0 || s->nheads <= 0 || s->headdim <= 0 || s->dstate <= 0 ||
      s->ngroups <= 0 || s->chunk <= 0 || (s->flags & ~SSD_DT_SOFTPLUS) != 0)
    return SSD_ERR_INVALID_ARGUMENT;
  if (s->dtype != SSD_F32 && s->dtype != SSD_BF16 && s->dtype != SSD_FP8) return SSD_ERR_INVALID_ARGUMENT;
  if (s->nheads % s->ngroups != 0) return SSD_ERR_INVALID_ARGUMENT;
  // Grid dimensions and 32-bit index products used inside the kernels.  Every
  // size is bounded first, so none of the products below can overflow.
  const int64_t sizes[] = {s->batch, s->seqlen, s->nheads, s->headdim, s->dstate, s->ngroups, s->chunk};
  for (int64_t v : sizes)
    if (v > INT32_MAX) return SSD_ERR_INVALID_ARGUMENT;
  const int64_t K = (s->seqlen + s->chunk - 1) / s->chunk;
  if (s->nheads > 65535 || s->batch * s->nheads > 65535 || s->batch * s->seqlen > INT32_MAX / 4 ||
      s->batch * K > INT32_MAX / s->nheads)
    return SSD_ERR_INVALID_ARGUMENT;
  if (!is_supported(s->dtype, s->chunk, s->headdim, s->dstate)) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

// Workspace layout of one chunked problem: b sequences of K whole chunks
// whose rows sit at row stride L (L >= K * Q).
Layout make_layout(const ssd_shape* s, int64_t L, int64_t K) {
  Layout y{};
  y.b = s->batch; y.L = L; y.H = s->nheads; y.P = s->headdim; y.N = s->dstate;
  y.G = s->ngroups; y.Q = s->chunk; y.K = K;
  y.esz = s->dtype == SSD_F32 ? 4 : 2;  // states, tiles, y, dt: bf16 unless fp32
  const int64_t nt = y.Q / 16;
  y.wtiles = nt * (nt + 1) / 2;
  const size_t states = (size_t)(y.b * y.K * y.H * y.P * y.N);
  size_t o = 0;
  y.cs_off = o;   o += align_up((size_t)(y.b * y.H * y.K * y.Q) * 4);
  y.hin_off = o;  o += align_up(states * y.esz);
  y.saved_bytes = o;
  o = 0;
  y.s_off = o;    o += align_up(states * y.esz);
  y.wt_off = o;   o += align_up((size_t)(y.b * y.K * y.G * y.wtiles * 256) * y.esz);
  y.fwd_bytes = o;
  o = 0;
  y.dhloc_off = o;  o += align_up(states * y.esz);
  y.g_off = o;      o += align_up(states * y.esz);
  // Head slices of the group-level backward launch (dW and the dC / dB head
  // sums; each slice writes fp32 partials that are summed in a fixed order):
  // about `target` workgroups per kind of block, never finer than one head and
  // never more than kMaxHeadSlices.  Measured at the 2.7B shape
  // (b*K*G*Q/64 = 256): two slices is fastest; more slices cost more in partial sums than the extra parallelism
  // gains, one slice starves dW.  Small problems (a one-chunk tail) would ask
  // for dozens of slices, whose serial partial sums on few workgroups cost far
  // more than the heads they spread.
  auto slices = [&](int64_t target) {
    const int64_t base = y.b * y.K * y.G * (y.Q / 64);
    const int64_t hpg = y.H / y.G;
    int64_t sl = (target + base - 1) / base;
    if (sl > kMaxHeadSlices) sl = kMaxHeadSlices;
    if (sl > hpg) sl = hpg;
    if (sl < 1) sl = 1;
    // the kernels give each slice ceil(hpg / sl) heads; take the slice count
    // that this covers exactly, so no slice is empty (9 heads in 4 slices of 3
    // would leave the last with none, and its loads would run past the group)
    const int64_t per = (hpg + sl - 1) / sl;
    return (hpg + per - 1) / per;
  };
  y.nslice = slices(512);
  y.dw_off = o;     o += align_up((size_t)(y.nslice * y.b * y.K * y.G * y.Q * y.Q) * 4);
  y.dcpart_off = o; o += align_up((size_t)(y.nslice * y.b * y.K * y.Q * y.G * y.N) * 4);
  y.dbpart_off = o; o += align_up((size_t)(y.nslice * y.b * y.K * y.Q * y.G * y.N) * 4);
  y.dapart_off = o; o += align_up((size_t)(y.b * y.K * y.H) * 4);
  y.ddpart_off = o; o += align_up((size_t)(y.b * y.K * y.H) * 4);
  const int64_t nsp = scan_bwd_splits((int)y.Q);
  y.dlpart_off = o; o += align_up((size_t)(y.b * y.K * y.H * dl_rows((int)y.Q) * y.Q) * 4);
  y.dlscal_off = o; o += align_up((size_t)(y.b * y.K * y.H * (nsp + 1)) * 4);
  y.bwd_bytes = o;
  return y;
}

// A sequence of L tokens runs as K = ceil(L / Q) chunks.  The whole ones
// are read and written in place; when L % Q = Lr > 0, the last one (chunk kf
// = L / Q) holds Lr tokens and runs on zero-padded copies of Q rows per
// sequence: the x, B, C copies are made by the forward and kept in the saved
// workspace (dt's only feeds the cumsum), dy's copy and the last chunk's
// outputs live in the backward scratch, and the valid rows are copied back
// to the caller's tensors.  The float32 step the cumsum writes ([b][H][K][Q],
// like cs) is saved for the backward.
// With SSD_DT_SOFTPLUS the backward adds per-chunk partials of the bias
// gradient.
struct Plan {
  Layout lay;
  int64_t kf, Lr;
  size_t sv_tx, sv_tB, sv_tC, sv_dtf, saved_bytes;
  size_t fw_tdt, fw_ty, fwd_bytes;
  size_t bw_tdy, bw_tdx, bw_tddt, bw_tdB, bw_tdC, bw_dbias, bwd_bytes;
};

Plan make_plan(const ssd_shape* s) {
  Plan p{};
  const int64_t Q = s->chunk, L = s->seqlen;
  p.kf = L / Q;
  p.Lr = L % Q;
  p.lay = make_layout(s, L, (L + Q - 1) / Q);
  const bool tail = p.Lr > 0;
  const size_t esz = s->dtype == SSD_F32 ? 4 : 2;                          // dt, y, dy, dx, ddt
  const size_t eszx = s->dtype == SSD_F32 ? 4 : (s->dtype == SSD_FP8 ? 1 : 2);  // x, B, C
  const size_t b = s->batch, H = s->nheads, P = s->headdim, N = s->dstate, G = s->ngroups, q = Q;
  const size_t xrows = tail ? align_up(b * q * H * P * eszx) : 0, trows = tail ? align_up(b * q * H * esz) : 0;
  const size_t yrows = tail ? align_up(b * q * H * P * esz) : 0;
  const size_t brows = tail ? align_up(b * q * G * N * eszx) : 0;   // B, C rows as stored
  const size_t grows = tail ? align_up(b * q * G * N * esz) : 0;    // dB, dC rows (bf16 also in FP8 mode)
  size_t o = p.lay.saved_bytes;
  p.sv_tx = o;   o += xrows;
  p.sv_tB = o;   o += brows;
  p.sv_tC = o;   o += brows;
  p.sv_dtf = o;  o += align_up(b * H * (size_t)p.lay.K * q * 4);
  p.saved_bytes = o;
  const bool sp = (s->flags & SSD_DT_SOFTPLUS) != 0;
  o = p.lay.fwd_bytes;
  p.fw_tdt = o; o += trows;
  p.fw_ty = o;  o += yrows;
  p.fwd_bytes = o;
  o = p.lay.bwd_bytes;
  p.bw_tdy = o;  o += yrows;
  p.bw_tdx = o;  o += yrows;
  p.bw_tddt = o; o += trows;
  p.bw_tdB = o;  o += grows;
  p.bw_tdC = o;  o += grows;
  p.bw_dbias = o; if (sp) o += align_up(b * (size_t)p.lay.K * H * 4);
  p.bwd_bytes = o;
  return p;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename P>
P* at(void* base, size_t off) { return reinterpret_cast<P*>(static_cast<char*>(base) + off); }
template <typename P>
const P* at(const void* base, size_t off) { return reinterpret_cast<const P*>(static_cast<const char*>(base) + off); }

// Workspace pointers of one problem: saved and scratch are the bases of its
// own regions.
void set_fwd_ws(FwdArgs& a, const Layout& lay, void* saved, void* scratch) {
  a.cs = at<float>(saved, lay.cs_off);
  a.hin = at<char>(saved, lay.hin_off);
  a.wt = at<char>(scratch, lay.wt_off);
  a.S = at<char>(scratch, lay.s_off);
}

void set_bwd_ws(BwdArgs& a, const Layout& lay, const void* saved, void* scratch) {
  a.cs = at<float>(saved, lay.cs_off);
  a.hin = at<char>(saved, lay.hin_off);
  a.dhloc = at<char>(scratch, lay.dhloc_off);
  a.gst = at<char>(scratch, lay.g_off);
  a.dw = at<float>(scratch, lay.dw_off);
  a.dcpart = at<float>(scratch, lay.dcpart_off);
  a.dbpart = at<float>(scratch, lay.dbpart_off);
  a.dapart = at<float>(scratch, lay.dapart_off);
  a.ddpart = at<float>(scratch, lay.ddpart_off);
  a.dlpart = at<float>(scratch, lay.dlpart_off);
  a.dlscal = at<float>(scratch, lay.dlscal_off);
}

bool dispatch_fwd(int dtype, const Layout& lay, const FwdArgs& a, hipStream_t stream, const ssd_probe* probe) {
#define SSD_DISPATCH(TT, TI, Q_, P_, N_)                    \
  if (lay.Q == Q_ && lay.P == P_ && lay.N == N_) {          \
    run_fwd<TT, TI, Q_, P_, N_>(lay, a, stream, probe);     \
    return true;                                            \
  }
#define SSD_DISPATCH_BF16(Q_, P_, N_) SSD_DISPATCH(bf16, bf16, Q_, P_, N_)
#define SSD_DISPATCH_FP8(Q_, P_, N_) SSD_DISPATCH(bf16, fp8, Q_, P_, N_)
#define SSD_DISPATCH_F32(Q_, P_, N_) SSD_DISPATCH(float, float, Q_, P_, N_)
  if (dtype == SSD_BF16) { SSD_BF16_CONFIGS(SSD_DISPATCH_BF16) }
  else if (dtype == SSD_FP8) { SSD_BF16_CONFIGS(SSD_DISPATCH_FP8) }
  else { SSD_F32_CONFIGS(SSD_DISPATCH_F32) }
#undef SSD_DISPATCH
#undef SSD_DISPATCH_BF16
#undef SSD_DISPATCH_FP8
#undef SSD_DISPATCH_F32
  return false;
}

bool dispatch_bwd(int dtype, const Layout& lay, const BwdArgs& a, hipStream_t stream, const ssd_probe* probe) {
#define SSD_DISPATCH(TT, TI, Q_, P_, N_)                    \
  if (lay.Q == Q_ && lay.P == P_ && lay.N == N_) {          \
    run_bwd<TT, TI, Q_, P_, N_>(lay, a, stream, probe);     \
    return true;                                            \
  }
#define SSD_DISPATCH_BF16(Q_, P_, N_) SSD_DISPATCH(bf16, bf16, Q_, P_, N_)
#define SSD_DISPATCH_FP8(Q_, P_, N_) SSD_DISPATCH(bf16, fp8, Q_, P_, N_)
#define SSD_DISPATCH_F32(Q_, P_, N_) SSD_DISPATCH(float, float, Q_, P_, N_)
  if (dtype == SSD_BF16) { SSD_BF16_CONFIGS(SSD_DISPATCH_BF16) }
  else if (dtype == SSD_FP8) { SSD_BF16_CONFIGS(SSD_DISPATCH_FP8) }
  else { SSD_F32_CONFIGS(SSD_DISPATCH_F32) }
#undef SSD_DISPATCH
#undef SSD_DISPATCH_BF16
#undef SSD_DISPATCH_FP8
#undef SSD_DISPATCH_F32
  return false;
}

}  // namespace
}  // namespace ssd

namespace ssd {
namespace {

// Argument checks of ssd_fwd other than its scratch (nothing is launched).
ssd_status check_fwd(const ssd_shape* s, const void* x, const void* dt, const float* A, const void* B, const void* C,
                     const float* D, const float* dt_bias, const float* initial_state, const void* y,
                     const float* final_state, const void* saved_ws, size_t saved_ws_bytes) {
  const ssd_status st = check_shape(s);
  if (st != SSD_OK) return st;
  if (!x || !dt || !A || !B || !C || !D || !y) return SSD_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x, dt, A, B, C, D, y, saved_ws, final_state, initial_state, dt_bias};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSD_ERR_INVALID_ARGUMENT;
  if (!saved_ws || saved_ws_bytes < make_plan(s).saved_bytes) return SSD_ERR_WORKSPACE;
  return SSD_OK;
}

// The forward's launches, after every check has passed.
ssd_status fwd_launch(const ssd_shape* s, const void* x, const void* dt, const float* A, const void* B, const void* C,
                      const float* D, const float* dt_bias, const float* initial_state, void* y, float* final_state,
                      void* saved_ws, size_t saved_ws_bytes, ssd_saved* saved_out, void* scratch,
                      hipStream_t stream, const ssd_probe* probe) {
  const Plan pl = make_plan(s);

  const int64_t esz = s->dtype == SSD_F32 ? 4 : 2;                          // dt, y
  const int64_t eszx = s->dtype == SSD_F32 ? 4 : (s->dtype == SSD_FP8 ? 1 : 2);  // x, B, C
  const int64_t b = s->batch, L = s->seqlen, Q = s->chunk, H = s->nheads, G = s->ngroups;
  const int64_t P = s->headdim, N = s->dstate;
  FwdArgs a{};
  a.x = x; a.dt = dt; a.B = B; a.C = C; a.A = A; a.D = D; a.y = y;
  a.init = initial_state;
  a.final_state = final_state;
  a.softplus = (s->flags & SSD_DT_SOFTPLUS) ? 1 : 0;
  a.dt_bias = dt_bias;
  a.dtf = at<float>(saved_ws, pl.sv_dtf);
  a.rows.L = L;
  a.rows.kf = (int)pl.kf;
  a.rows.lr = (int)pl.Lr;
  set_fwd_ws(a, pl.lay, saved_ws, scratch);
  if (pl.Lr > 0) {
    a.rows.x = at<char>(saved_ws, pl.sv_tx);
    a.rows.dt = at<char>(scratch, pl.fw_tdt);
    a.rows.B = at<char>(saved_ws, pl.sv_tB);
    a.rows.C = at<char>(saved_ws, pl.sv_tC);
    a.rows.y = at<char>(scratch, pl.fw_ty);
    const RowCopy in{{x, dt, B, C},
                     {const_cast<void*>(a.rows.x), const_cast<void*>(a.rows.dt), const_cast<void*>(a.rows.B),
                      const_cast<void*>(a.rows.C)},
                     {H * P * eszx, H * esz, G * N * eszx, G * N * eszx}, 4};
    pad_rows(in, L, pl.kf * Q, pl.Lr, Q, b, stream);
  }
  dispatch_fwd(s->dtype, pl.lay, a, stream, probe);
  if (pl.Lr > 0) {
    const RowCopy out{{a.rows.y}, {y}, {H * P * esz}, 1};
    unpad_rows(out, L, pl.kf * Q, pl.Lr, Q, b, stream);
  }
  if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;

  if (saved_out) {
    saved_out->shape = *s;
    saved_out->x = x; saved_out->dt = dt; saved_out->B = B; saved_out->C = C;
    saved_out->A = A; saved_out->D = D;
    saved_out->saved_ws = saved_ws;
    saved_out->saved_ws_bytes = saved_ws_bytes;
  }
  return SSD_OK;
}

// Device address of `scratch` on the GPU that `stream` runs on, which must be
// the current device (hipGetSymbolAddress resolves the current device's copy).
// Looked up once per device with that device current and kept; the lookup is
// the only state the library keeps, written once per device under a lock.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];

ssd_status static_scratch(hipStream_t stream, void** out) {
  int cur = -1, sdev = -1;
  if (hipGetDevice(&cur) != hipSuccess) return SSD_ERR_HIP;
  if (stream) {
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return SSD_ERR_HIP;
    if (sdev != cur) return SSD_ERR_INVALID_ARGUMENT;
  }
  if (cur < 0 || cur >= kMaxDevices) return SSD_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[cur]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSD_ERR_HIP;
    g_scratch_dev[cur] = p;
  }
  *out = g_scratch_dev[cur];
  return SSD_OK;
}

}  // namespace
}  // namespace ssd

using namespace ssd;

extern "C" {

const char* ssd_version(void) { return "0.1.0"; }

const char* ssd_status_string(int32_t st) {
  switch (st) {
    case SSD_OK: return "ok";
    case SSD_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SSD_ERR_UNSUPPORTED: return "unsupported (dtype, chunk, headdim, dstate) combination";
    case SSD_ERR_WORKSPACE: return "workspace missing or too small";
    case SSD_ERR_HIP: return "HIP error";
    case SSD_ERR_TOO_LARGE:
      return "problem too large for ssd_fwd_noalloc: its forward scratch exceeds the library's static buffer "
             "(SSD_FWD_STATIC_SCRATCH_BYTES); use ssd_fwd with a caller-allocated scratch";
  }
  return "unknown status";
}

const char* ssd_kernel_name(int32_t k) {
  static const char* names[SSD_NUM_KERNELS] = {
      "cumsum_bmm", "chunk_state", "state_passing", "chunk_scan",
      "chunk_state_bwd", "state_passing_bwd", "chunk_scan_bwd", "dw_heads", "bc_final", "da_dd"};
  if (k < 0 || k >= SSD_NUM_KERNELS) return nullptr;
  return names[k];
}

ssd_status ssd_check_shape(const ssd_shape* s) { return check_shape(s); }

size_t ssd_saved_bytes(const ssd_shape* s) { return check_shape(s) == SSD_OK ? make_plan(s).saved_bytes : 0; }
size_t ssd_fwd_scratch_bytes(const ssd_shape* s) { return check_shape(s) == SSD_OK ? make_plan(s).fwd_bytes : 0; }
size_t ssd_bwd_scratch_bytes(const ssd_shape* s) { return check_shape(s) == SSD_OK ? make_plan(s).bwd_bytes : 0; }

ssd_status ssd_workspace_regions(const ssd_shape* s, ssd_regions* out) {
  if (!out) return SSD_ERR_INVALID_ARGUMENT;
  const ssd_status st = check_shape(s);
  if (st != SSD_OK) return st;
  const Plan p = make_plan(s);
  out->cs = p.lay.cs_off;
  out->step = p.sv_dtf;
  out->hin = p.lay.hin_off;
  out->chunk_state = p.lay.s_off;
  out->dhloc = p.lay.dhloc_off;
  out->gstate = p.lay.g_off;
  return SSD_OK;
}

ssd_status ssd_fwd(const ssd_shape* s, const void* x, const void* dt, const float* A, const void* B, const void* C,
                   const float* D, const float* dt_bias, const float* initial_state, void* y, float* final_state, void* saved_ws,
                   size_t saved_ws_bytes, ssd_saved* saved_out, void* scratch, size_t scratch_bytes,
                   hipStream_t stream, const ssd_probe* probe) {
  const ssd_status st = check_fwd(s, x, dt, A, B, C, D, dt_bias, initial_state, y, final_state, saved_ws,
                                  saved_ws_bytes);
  if (st != SSD_OK) return st;
  if (!scratch || !aligned16(scratch)) return scratch ? SSD_ERR_INVALID_ARGUMENT : SSD_ERR_WORKSPACE;
  if (scratch_bytes < make_plan(s).fwd_bytes) return SSD_ERR_WORKSPACE;
  return fwd_launch(s, x, dt, A, B, C, D, dt_bias, initial_state, y, final_state, saved_ws, saved_ws_bytes,
                    saved_out, scratch, stream, probe);
}

ssd_status ssd_fwd_noalloc(const ssd_shape* s, const void* x, const void* dt, const float* A, const void* B,
                           const void* C, const float* D, const float* dt_bias, const float* initial_state, void* y,
                           float* final_state, void* saved_ws, size_t saved_ws_bytes, ssd_saved* saved_out,
                           hipStream_t stream, const ssd_probe* probe) {
  const ssd_status st = check_fwd(s, x, dt, A, B, C, D, dt_bias, initial_state, y, final_state, saved_ws,
                                  saved_ws_bytes);
  if (st != SSD_OK) return st;
  if (make_plan(s).fwd_bytes > (size_t)SSD_FWD_STATIC_SCRATCH_BYTES) return SSD_ERR_TOO_LARGE;
  void* scr = nullptr;
  const ssd_status ss = static_scratch(stream, &scr);
  if (ss != SSD_OK) return ss;
  // nothing in the forward scratch needs to start at zero: the chunk states
  // are written before they are read, the padded step rows of a shorter last
  // chunk are written whole by the padding launch and its y rows by the scan
  return fwd_launch(s, x, dt, A, B, C, D, dt_bias, initial_state, y, final_state, saved_ws, saved_ws_bytes,
                    saved_out, scr, stream, probe);
}

ssd_status ssd_bwd(const ssd_saved* sv, const void* dy, const float* dfinal_state, void* dx, void* ddt, float* dA,
                   void* dB, void* dC, float* dD, float* ddt_bias, float* dinitial_state, void* scratch, size_t scratch_bytes,
                   hipStream_t stream, const ssd_probe* probe) {
  if (!sv) return SSD_ERR_INVALID_ARGUMENT;
  const ssd_shape* s = &sv->shape;
  const ssd_status st = check_shape(s);
  if (st != SSD_OK) return st;
  if (!sv->x || !sv->dt || !sv->A || !sv->B || !sv->C || !sv->D || !dy || !dx || !ddt || !dA || !dB || !dC || !dD)
    return SSD_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {sv->x, sv->dt, sv->A, sv->B, sv->C, sv->D, dy, dx, ddt, dA, dB, dC, dD, sv->saved_ws, scratch,
                        dfinal_state, dinitial_state, ddt_bias};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSD_ERR_INVALID_ARGUMENT;
  const Plan pl = make_plan(s);
  if (!sv->saved_ws || sv->saved_ws_bytes < pl.saved_bytes) return SSD_ERR_WORKSPACE;
  if (!scratch || scratch_bytes < pl.bwd_bytes) return SSD_ERR_WORKSPACE;

  const size_t esz = s->dtype == SSD_F32 ? 4 : 2;  // dy, dx, ddt, dB, dC (bf16 also in FP8 mode)
  const int64_t b = s->batch, L = s->seqlen, Q = s->chunk, H = s->nheads, G = s->ngroups;
  const int64_t P = s->headdim, N = s->dstate;
  BwdArgs a{};
  a.x = sv->x; a.dt = sv->dt; a.B = sv->B; a.C = sv->C; a.dy = dy; a.A = sv->A; a.D = sv->D;
  a.dx = dx; a.ddt = ddt; a.dB = dB; a.dC = dC; a.dA = dA; a.dD = dD;
  a.dfinal = dfinal_state; a.dinit = dinitial_state;
  a.dtf = at<float>(sv->saved_ws, pl.sv_dtf);
  a.softplus = (s->flags & SSD_DT_SOFTPLUS) ? 1 : 0;
  if (a.softplus) {
    a.ddt_bias = ddt_bias;
    a.dbiaspart = at<float>(scratch, pl.bw_dbias);
  }
  a.rows.L = L;
  a.rows.kf = (int)pl.kf;
  a.rows.lr = (int)pl.Lr;
  set_bwd_ws(a, pl.lay, sv->saved_ws, scratch);
  if (pl.Lr > 0) {
    a.rows.x = at<char>(sv->saved_ws, pl.sv_tx);
    a.rows.B = at<char>(sv->saved_ws, pl.sv_tB);
    a.rows.C = at<char>(sv->saved_ws, pl.sv_tC);
    a.rows.dy = at<char>(scratch, pl.bw_tdy);
    a.rows.dx = at<char>(scratch, pl.bw_tdx);
    a.rows.ddt = at<char>(scratch, pl.bw_tddt);
    a.rows.dB = at<char>(scratch, pl.bw_tdB);
    a.rows.dC = at<char>(scratch, pl.bw_tdC);
    const RowCopy in{{dy}, {const_cast<void*>(a.rows.dy)}, {H * P * (int64_t)esz}, 1};
    pad_rows(in, L, pl.kf * Q, pl.Lr, Q, b, stream);
  }
  dispatch_bwd(s->dtype, pl.lay, a, stream, probe);
  if (pl.Lr > 0) {
    const RowCopy out{{a.rows.dx, a.rows.ddt, a.rows.dB, a.rows.dC},
                      {dx, ddt, dB, dC},
                      {H * P * (int64_t)esz, H * (int64_t)esz, G * N * (int64_t)esz, G * N * (int64_t)esz}, 4};
    unpad_rows(out, L, pl.kf * Q, pl.Lr, Q, b, stream);
  }
  if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
  return SSD_OK;
}

// ---- causal depthwise conv1d

namespace {
ssd_status conv_check(const ssd_conv_shape* s) {
  if (!s) return SSD_ERR_INVALID_ARGUMENT;
  if (s->batch <= 0 || s->seqlen <= 0 || s->channels <= 0 || s->reserved != 0) return SSD_ERR_INVALID_ARGUMENT;
  if (s->dtype != SSD_F32 && s->dtype != SSD_BF16) return SSD_ERR_INVALID_ARGUMENT;
  if (s->silu != 0 && s->silu != 1) return SSD_ERR_INVALID_ARGUMENT;
  if (s->batch > 65535 || s->seqlen > INT32_MAX || s->channels > INT32_MAX / 8 || s->batch * s->seqlen > INT32_MAX)
    return SSD_ERR_INVALID_ARGUMENT;
  if (s->width < 2 || s->width > 4 || s->channels % 4 != 0) return SSD_ERR_UNSUPPORTED;
  // one workgroup row per block of run blocks (grid y)
  if (conv_partial_rows(s->batch, s->seqlen, s->dtype == SSD_BF16 ? 2 : 4) > 65535) return SSD_ERR_INVALID_ARGUMENT;
  return SSD_OK;
}

ConvArgs conv_args(const ssd_conv_shape* s) {
  ConvArgs a{};
  a.b = s->batch; a.L = s->seqlen; a.C = s->channels;
  a.W = s->width; a.esz = s->dtype == SSD_BF16 ? 2 : 4; a.silu = s->silu;
  return a;
}
}  // namespace

ssd_status ssd_conv1d_check_shape(const ssd_conv_shape* s) { return conv_check(s); }

size_t ssd_conv1d_bwd_scratch_bytes(const ssd_conv_shape* s) {
  if (conv_check(s) != SSD_OK) return 0;
  const int esz = s->dtype == SSD_BF16 ? 2 : 4;
  return align_up((size_t)conv_partial_rows(s->batch, s->seqlen, esz) * s->channels * (s->width + 1) * 4);
}

ssd_status ssd_conv1d_fwd(const ssd_conv_shape* s, const void* x, const float* w, const float* bias,
                          const void* x_prev, void* y, hipStream_t stream) {
  const ssd_status st = conv_check(s);
  if (st != SSD_OK) return st;
  if (!x || !w || !y) return SSD_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x, w, bias, x_prev, y};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSD_ERR_INVALID_ARGUMENT;
  ConvArgs a = conv_args(s);
  a.x = x; a.w = w; a.bias = bias; a.x_prev = x_prev; a.y = y;
  run_conv_fwd(a, stream);
  return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

ssd_status ssd_conv1d_bwd(const ssd_conv_shape* s, const void* x, const float* w, const float* bias,
                          const void* x_prev, const void* dy, void* dx, float* dw, float* dbias, void* dx_prev,
                          void* scratch, size_t scratch_bytes, hipStream_t stream) {
  const ssd_status st = conv_check(s);
  if (st != SSD_OK) return st;
  if (!x || !w || !dy || !dx || !dw) return SSD_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x, w, bias, x_prev, dy, dx, dw, dbias, dx_prev, scratch};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSD_ERR_INVALID_ARGUMENT;
  if (!scratch || scratch_bytes < ssd_conv1d_bwd_scratch_bytes(s)) return SSD_ERR_WORKSPACE;
  ConvArgs a = conv_args(s);
  a.x = x; a.w = w; a.bias = bias; a.x_prev = x_prev; a.dy = dy;
  a.dx = dx; a.dw = dw; a.dbias = dbias; a.dx_prev = dx_prev;
  a.part = static_cast<float*>(scratch);
  run_conv_bwd(a, stream);
  return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // extern "C"
