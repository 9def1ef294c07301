// C-ABI entry points of libssd: argument checks, workspace layout and
// dispatch to the compiled (dtype, chunk, headdim, dstate) instantiations.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "kernels.h"

namespace ssd {
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool is_supported(int dtype, int64_t Q, int64_t P, int64_t N) {
#define SSD_MATCH(Q_, P_, N_) if (Q == Q_ && P == P_ && N == N_) return true;
  if (dtype == SSD_BF16) { SSD_BF16_CONFIGS(SSD_MATCH) }
  if (dtype == SSD_F32) { SSD_F32_CONFIGS(SSD_MATCH) }
#undef SSD_MATCH
  return false;
}

ssd_status check_shape(const ssd_shape* s) {
  if (!s) return SSD_ERR_INVALID_ARGUMENT;
  if (s->batch <= 0 || s->seqlen <= 0 || s->nheads <= 0 || s->headdim <= 0 || s->dstate <= 0 ||
      s->ngroups <= 0 || s->chunk <= 0 || s->reserved != 0)
    return SSD_ERR_INVALID_ARGUMENT;
  if (s->dtype != SSD_F32 && s->dtype != SSD_BF16) return SSD_ERR_INVALID_ARGUMENT;
  if (s->nheads % s->ngroups != 0) return SSD_ERR_INVALID_ARGUMENT;
  // Grid dimensions and 32-bit index products used inside the kernels.
  const int64_t K = (s->seqlen + s->chunk - 1) / s->chunk;
  if (s->batch * K * s->nheads > INT32_MAX || s->batch * s->nheads > 65535 ||
      s->batch * s->seqlen > INT32_MAX / 4 || s->nheads > 65535)
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
  y.esz = s->dtype == SSD_BF16 ? 2 : 4;
  const int64_t nt = y.Q / 16;
  y.wtiles = nt * (nt + 1) / 2;
  const size_t states = (size_t)(y.b * y.K * y.H * y.P * y.N);
  size_t o = 0;
  y.cs_off = o;   o += align_up((size_t)(y.b * y.H * y.K * y.Q) * 4);
  y.hin_off = o;  o += align_up(states * y.esz);
  y.wt_off = o;   o += align_up((size_t)(y.b * y.K * y.G * y.wtiles * 256) * y.esz);
  y.wtb_off = o;  o += align_up((size_t)(y.b * y.K * y.G * y.wtiles * 256) * y.esz);
  y.saved_bytes = o;
  o = 0;
  y.s_off = o;    o += align_up(states * 4);
  y.fwd_bytes = o;
  o = 0;
  y.dhloc_off = o;  o += align_up(states * 4);
  y.g_off = o;      o += align_up(states * y.esz);
  // Head slices for the group-level backward kernels (each slice writes an
  // fp32 partial that is summed in a fixed order): about `target` workgroups
  // per launch, never finer than one head.  Measured at the 2.7B shape
  // (b*K*G*Q/64 = 256): two slices for both is fastest; more slices cost more
  // in partial sums than the extra parallelism gains, one slice starves dW.
  auto slices = [&](int64_t target) {
    const int64_t base = y.b * y.K * y.G * (y.Q / 64);
    const int64_t hpg = y.H / y.G;
    int64_t sl = (target + base - 1) / base;
    if (sl > hpg) sl = hpg;
    if (sl < 1) sl = 1;
    return sl;
  };
  y.nslice = slices(512);
  y.nslice_bc = slices(512);
  y.dw_off = o;     o += align_up((size_t)(y.nslice * y.b * y.K * y.G * y.Q * y.Q) * 4);
  y.dcpart_off = o; o += align_up((size_t)(y.nslice_bc * y.b * y.L * y.G * y.N) * 4);
  y.dbpart_off = o; o += align_up((size_t)(y.nslice_bc * y.b * y.L * y.G * y.N) * 4);
  y.dapart_off = o; o += align_up((size_t)(y.b * y.K * y.H) * 4);
  y.ddpart_off = o; o += align_up((size_t)(y.b * y.K * y.H) * 4);
  const int64_t nsp = scan_bwd_splits((int)y.Q);
  y.dlpart_off = o; o += align_up((size_t)(y.b * y.K * y.H * (nsp + 3) * y.Q) * 4);
  y.dlscal_off = o; o += align_up((size_t)(y.b * y.K * y.H * (nsp + 1)) * 4);
  y.bwd_bytes = o;
  return y;
}

// A sequence of L tokens runs as Kf = L / Q whole chunks in place (the
// "main" problem, row stride L) and, when Lr = L % Q > 0, its last Lr tokens
// as a one-chunk "tail" problem on zero-padded copies ([b][Q] rows, kept in
// the saved workspace for the inputs and in scratch for dy and the tail's
// outputs).  The tail starts from the state the main part leaves and returns
// the cotangent of that state, which seeds the main part's backward; the
// tail's dA / dD are added after the main part's chunk sums.
struct Plan {
  Layout main, tail;
  bool has_main, has_tail;
  int64_t Kf, Lr;
  // saved workspace
  size_t sv_main, sv_tail, sv_tx, sv_tdt, sv_tB, sv_tC, saved_bytes;
  // forward scratch
  size_t fw_main, fw_tail, fw_fsmid, fw_ty, fwd_bytes;
  // backward scratch
  size_t bw_main, bw_tail, bw_tdy, bw_tdx, bw_tddt, bw_tdB, bw_tdC, bw_tdA, bw_tdD, bw_tds0, bwd_bytes;
};

Plan make_plan(const ssd_shape* s) {
  Plan p{};
  const int64_t Q = s->chunk, L = s->seqlen;
  p.Kf = L / Q;
  p.Lr = L % Q;
  p.has_main = p.Kf > 0;
  p.has_tail = p.Lr > 0;
  if (p.has_main) p.main = make_layout(s, L, p.Kf);
  if (p.has_tail) p.tail = make_layout(s, Q, 1);
  const size_t esz = s->dtype == SSD_BF16 ? 2 : 4;
  const size_t b = s->batch, H = s->nheads, P = s->headdim, N = s->dstate, G = s->ngroups, q = Q;
  const size_t xrows = align_up(b * q * H * P * esz), trows = align_up(b * q * H * esz);
  const size_t brows = align_up(b * q * G * N * esz), state = align_up(b * H * P * N * 4);
  size_t o = 0;
  p.sv_main = o;  if (p.has_main) o += p.main.saved_bytes;
  p.sv_tail = o;  if (p.has_tail) o += p.tail.saved_bytes;
  p.sv_tx = o;    if (p.has_tail) o += xrows;
  p.sv_tdt = o;   if (p.has_tail) o += trows;
  p.sv_tB = o;    if (p.has_tail) o += brows;
  p.sv_tC = o;    if (p.has_tail) o += brows;
  p.saved_bytes = o;
  o = 0;
  p.fw_main = o;  if (p.has_main) o += p.main.fwd_bytes;
  p.fw_tail = o;  if (p.has_tail) o += p.tail.fwd_bytes;
  p.fw_fsmid = o; if (p.has_tail) o += state;
  p.fw_ty = o;    if (p.has_tail) o += xrows;
  p.fwd_bytes = o;
  o = 0;
  p.bw_main = o;  if (p.has_main) o += p.main.bwd_bytes;
  p.bw_tail = o;  if (p.has_tail) o += p.tail.bwd_bytes;
  p.bw_tdy = o;   if (p.has_tail) o += xrows;
  p.bw_tdx = o;   if (p.has_tail) o += xrows;
  p.bw_tddt = o;  if (p.has_tail) o += trows;
  p.bw_tdB = o;   if (p.has_tail) o += brows;
  p.bw_tdC = o;   if (p.has_tail) o += brows;
  p.bw_tdA = o;   if (p.has_tail) o += align_up(H * 4);
  p.bw_tdD = o;   if (p.has_tail) o += align_up(H * 4);
  p.bw_tds0 = o;  if (p.has_tail) o += state;
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
  a.wt = at<char>(saved, lay.wt_off);
  a.wtb = at<char>(saved, lay.wtb_off);
  a.S = at<float>(scratch, lay.s_off);
}

void set_bwd_ws(BwdArgs& a, const Layout& lay, const void* saved, void* scratch) {
  a.cs = at<float>(saved, lay.cs_off);
  a.hin = at<char>(saved, lay.hin_off);
  a.w = at<char>(saved, lay.wtb_off);
  a.dhloc = at<float>(scratch, lay.dhloc_off);
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
#define SSD_DISPATCH(TT, Q_, P_, N_)                        \
  if (lay.Q == Q_ && lay.P == P_ && lay.N == N_) {          \
    run_fwd<TT, Q_, P_, N_>(lay, a, stream, probe);         \
    return true;                                            \
  }
#define SSD_DISPATCH_BF16(Q_, P_, N_) SSD_DISPATCH(bf16, Q_, P_, N_)
#define SSD_DISPATCH_F32(Q_, P_, N_) SSD_DISPATCH(float, Q_, P_, N_)
  if (dtype == SSD_BF16) { SSD_BF16_CONFIGS(SSD_DISPATCH_BF16) }
  else { SSD_F32_CONFIGS(SSD_DISPATCH_F32) }
#undef SSD_DISPATCH
#undef SSD_DISPATCH_BF16
#undef SSD_DISPATCH_F32
  return false;
}

bool dispatch_bwd(int dtype, const Layout& lay, const BwdArgs& a, hipStream_t stream, const ssd_probe* probe) {
#define SSD_DISPATCH(TT, Q_, P_, N_)                        \
  if (lay.Q == Q_ && lay.P == P_ && lay.N == N_) {          \
    run_bwd<TT, Q_, P_, N_>(lay, a, stream, probe);         \
    return true;                                            \
  }
#define SSD_DISPATCH_BF16(Q_, P_, N_) SSD_DISPATCH(bf16, Q_, P_, N_)
#define SSD_DISPATCH_F32(Q_, P_, N_) SSD_DISPATCH(float, Q_, P_, N_)
  if (dtype == SSD_BF16) { SSD_BF16_CONFIGS(SSD_DISPATCH_BF16) }
  else { SSD_F32_CONFIGS(SSD_DISPATCH_F32) }
#undef SSD_DISPATCH
#undef SSD_DISPATCH_BF16
#undef SSD_DISPATCH_F32
  return false;
}

}  // namespace
}  // namespace ssd

using namespace ssd;

extern "C" {

const char* ssd_version(void) { return "0.1.0"; }

const char* ssd_status_string(ssd_status st) {
  switch (st) {
    case SSD_OK: return "ok";
    case SSD_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SSD_ERR_UNSUPPORTED: return "unsupported (dtype, chunk, headdim, dstate) combination";
    case SSD_ERR_WORKSPACE: return "workspace missing or too small";
    case SSD_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* ssd_kernel_name(int32_t k) {
  static const char* names[SSD_NUM_KERNELS] = {
      "chunk_cumsum", "bmm_fwd", "chunk_state", "state_passing", "chunk_scan",
      "chunk_state_bwd", "state_passing_bwd", "chunk_scan_bwd", "dw", "dc", "db", "da_dd"};
  if (k < 0 || k >= SSD_NUM_KERNELS) return nullptr;
  return names[k];
}

ssd_status ssd_check_shape(const ssd_shape* s) { return check_shape(s); }

size_t ssd_saved_bytes(const ssd_shape* s) { return check_shape(s) == SSD_OK ? make_plan(s).saved_bytes : 0; }
size_t ssd_fwd_scratch_bytes(const ssd_shape* s) { return check_shape(s) == SSD_OK ? make_plan(s).fwd_bytes : 0; }
size_t ssd_bwd_scratch_bytes(const ssd_shape* s) { return check_shape(s) == SSD_OK ? make_plan(s).bwd_bytes : 0; }

ssd_status ssd_fwd(const ssd_shape* s, const void* x, const void* dt, const float* A, const void* B, const void* C,
                   const float* D, const float* initial_state, void* y, float* final_state, void* saved_ws,
                   size_t saved_ws_bytes, ssd_saved* saved_out, void* scratch, size_t scratch_bytes,
                   hipStream_t stream, const ssd_probe* probe) {
  const ssd_status st = check_shape(s);
  if (st != SSD_OK) return st;
  if (!x || !dt || !A || !B || !C || !D || !y) return SSD_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x, dt, A, B, C, D, y, saved_ws, scratch};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSD_ERR_INVALID_ARGUMENT;
  if (final_state && !aligned16(final_state)) return SSD_ERR_INVALID_ARGUMENT;
  if (initial_state && !aligned16(initial_state)) return SSD_ERR_INVALID_ARGUMENT;
  const Plan pl = make_plan(s);
  if (!saved_ws || saved_ws_bytes < pl.saved_bytes) return SSD_ERR_WORKSPACE;
  if (!scratch || scratch_bytes < pl.fwd_bytes) return SSD_ERR_WORKSPACE;

  const size_t esz = s->dtype == SSD_BF16 ? 2 : 4;
  const int64_t b = s->batch, L = s->seqlen, Q = s->chunk, H = s->nheads, G = s->ngroups;
  const int64_t P = s->headdim, N = s->dstate;
  float* fs_mid = pl.has_tail ? at<float>(scratch, pl.fw_fsmid) : nullptr;
  if (pl.has_main) {
    FwdArgs a{};
    a.x = x; a.dt = dt; a.B = B; a.C = C; a.A = A; a.D = D; a.y = y;
    a.init = initial_state;
    a.final_state = pl.has_tail ? fs_mid : final_state;
    set_fwd_ws(a, pl.main, at<char>(saved_ws, pl.sv_main), at<char>(scratch, pl.fw_main));
    dispatch_fwd(s->dtype, pl.main, a, stream, probe);
  }
  if (pl.has_tail) {
    const int64_t row0 = pl.Kf * Q;
    void* tx = at<char>(saved_ws, pl.sv_tx);
    void* tdt = at<char>(saved_ws, pl.sv_tdt);
    void* tB = at<char>(saved_ws, pl.sv_tB);
    void* tC = at<char>(saved_ws, pl.sv_tC);
    void* ty = at<char>(scratch, pl.fw_ty);
    pad_rows(x, tx, H * P * esz, L, row0, pl.Lr, Q, b, stream);
    pad_rows(dt, tdt, H * esz, L, row0, pl.Lr, Q, b, stream);
    pad_rows(B, tB, G * N * esz, L, row0, pl.Lr, Q, b, stream);
    pad_rows(C, tC, G * N * esz, L, row0, pl.Lr, Q, b, stream);
    FwdArgs a{};
    a.x = tx; a.dt = tdt; a.B = tB; a.C = tC; a.A = A; a.D = D; a.y = ty;
    a.init = pl.has_main ? fs_mid : initial_state;
    a.final_state = final_state;
    set_fwd_ws(a, pl.tail, at<char>(saved_ws, pl.sv_tail), at<char>(scratch, pl.fw_tail));
    dispatch_fwd(s->dtype, pl.tail, a, stream, pl.has_main ? nullptr : probe);
    unpad_rows(ty, y, H * P * esz, L, row0, pl.Lr, Q, b, stream);
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

ssd_status ssd_bwd(const ssd_saved* sv, const void* dy, const float* dfinal_state, void* dx, void* ddt, float* dA,
                   void* dB, void* dC, float* dD, float* dinitial_state, void* scratch, size_t scratch_bytes,
                   hipStream_t stream, const ssd_probe* probe) {
  if (!sv) return SSD_ERR_INVALID_ARGUMENT;
  const ssd_shape* s = &sv->shape;
  const ssd_status st = check_shape(s);
  if (st != SSD_OK) return st;
  if (!sv->x || !sv->dt || !sv->A || !sv->B || !sv->C || !sv->D || !dy || !dx || !ddt || !dA || !dB || !dC || !dD)
    return SSD_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {sv->x, sv->dt, sv->A, sv->B, sv->C, sv->D, dy, dx, ddt, dA, dB, dC, dD, sv->saved_ws, scratch,
                        dfinal_state, dinitial_state};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSD_ERR_INVALID_ARGUMENT;
  const Plan pl = make_plan(s);
  if (!sv->saved_ws || sv->saved_ws_bytes < pl.saved_bytes) return SSD_ERR_WORKSPACE;
  if (!scratch || scratch_bytes < pl.bwd_bytes) return SSD_ERR_WORKSPACE;

  const size_t esz = s->dtype == SSD_BF16 ? 2 : 4;
  const int64_t b = s->batch, L = s->seqlen, Q = s->chunk, H = s->nheads, G = s->ngroups;
  const int64_t P = s->headdim, N = s->dstate;
  float* tds0 = pl.has_tail ? at<float>(scratch, pl.bw_tds0) : nullptr;
  float* tdA = pl.has_tail ? at<float>(scratch, pl.bw_tdA) : nullptr;
  float* tdD = pl.has_tail ? at<float>(scratch, pl.bw_tdD) : nullptr;
  // The tail goes first: its initial-state gradient is the main part's
  // final-state cotangent.
  if (pl.has_tail) {
    const int64_t row0 = pl.Kf * Q;
    void* tdy = at<char>(scratch, pl.bw_tdy);
    void* tdx = at<char>(scratch, pl.bw_tdx);
    void* tddt = at<char>(scratch, pl.bw_tddt);
    void* tdB = at<char>(scratch, pl.bw_tdB);
    void* tdC = at<char>(scratch, pl.bw_tdC);
    pad_rows(dy, tdy, H * P * esz, L, row0, pl.Lr, Q, b, stream);
    BwdArgs a{};
    a.x = at<char>(sv->saved_ws, pl.sv_tx); a.dt = at<char>(sv->saved_ws, pl.sv_tdt);
    a.B = at<char>(sv->saved_ws, pl.sv_tB); a.C = at<char>(sv->saved_ws, pl.sv_tC);
    a.dy = tdy; a.A = sv->A; a.D = sv->D;
    a.dx = tdx; a.ddt = tddt; a.dB = tdB; a.dC = tdC;
    a.dA = pl.has_main ? tdA : dA; a.dD = pl.has_main ? tdD : dD;
    a.dfinal = dfinal_state;
    a.dinit = pl.has_main ? tds0 : dinitial_state;
    set_bwd_ws(a, pl.tail, at<char>(sv->saved_ws, pl.sv_tail), at<char>(scratch, pl.bw_tail));
    dispatch_bwd(s->dtype, pl.tail, a, stream, pl.has_main ? nullptr : probe);
    unpad_rows(tdx, dx, H * P * esz, L, row0, pl.Lr, Q, b, stream);
    unpad_rows(tddt, ddt, H * esz, L, row0, pl.Lr, Q, b, stream);
    unpad_rows(tdB, dB, G * N * esz, L, row0, pl.Lr, Q, b, stream);
    unpad_rows(tdC, dC, G * N * esz, L, row0, pl.Lr, Q, b, stream);
  }
  if (pl.has_main) {
    BwdArgs a{};
    a.x = sv->x; a.dt = sv->dt; a.B = sv->B; a.C = sv->C; a.dy = dy; a.A = sv->A; a.D = sv->D;
    a.dx = dx; a.ddt = ddt; a.dB = dB; a.dC = dC; a.dA = dA; a.dD = dD;
    a.dfinal = pl.has_tail ? tds0 : dfinal_state;
    a.dinit = dinitial_state;
    a.dA_add = tdA; a.dD_add = tdD;
    set_bwd_ws(a, pl.main, at<char>(sv->saved_ws, pl.sv_main), at<char>(scratch, pl.bw_main));
    dispatch_bwd(s->dtype, pl.main, a, stream, probe);
  }
  if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
  return SSD_OK;
}

}  // extern "C"
