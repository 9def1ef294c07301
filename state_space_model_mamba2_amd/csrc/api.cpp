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
  if (s->nheads % s->ngroups != 0 || s->seqlen % s->chunk != 0) return SSD_ERR_INVALID_ARGUMENT;
  // Grid dimensions and 32-bit index products used inside the kernels.
  const int64_t K = s->seqlen / s->chunk;
  if (s->batch * K * s->nheads > INT32_MAX || s->batch * s->nheads > 65535 ||
      s->batch * s->seqlen > INT32_MAX / 4 || s->nheads > 65535)
    return SSD_ERR_INVALID_ARGUMENT;
  if (!is_supported(s->dtype, s->chunk, s->headdim, s->dstate)) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

Layout make_layout(const ssd_shape* s) {
  Layout y{};
  y.b = s->batch; y.L = s->seqlen; y.H = s->nheads; y.P = s->headdim; y.N = s->dstate;
  y.G = s->ngroups; y.Q = s->chunk; y.K = s->seqlen / s->chunk;
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

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename P>
P* at(void* base, size_t off) { return reinterpret_cast<P*>(static_cast<char*>(base) + off); }
template <typename P>
const P* at(const void* base, size_t off) { return reinterpret_cast<const P*>(static_cast<const char*>(base) + off); }

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

size_t ssd_saved_bytes(const ssd_shape* s) { return check_shape(s) == SSD_OK ? make_layout(s).saved_bytes : 0; }
size_t ssd_fwd_scratch_bytes(const ssd_shape* s) { return check_shape(s) == SSD_OK ? make_layout(s).fwd_bytes : 0; }
size_t ssd_bwd_scratch_bytes(const ssd_shape* s) { return check_shape(s) == SSD_OK ? make_layout(s).bwd_bytes : 0; }

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
  const Layout lay = make_layout(s);
  if (!saved_ws || saved_ws_bytes < lay.saved_bytes) return SSD_ERR_WORKSPACE;
  if (!scratch || scratch_bytes < lay.fwd_bytes) return SSD_ERR_WORKSPACE;

  FwdArgs a{};
  a.x = x; a.dt = dt; a.B = B; a.C = C; a.A = A; a.D = D; a.y = y; a.final_state = final_state;
  a.init = initial_state;
  a.cs = at<float>(saved_ws, lay.cs_off);
  a.hin = at<char>(saved_ws, lay.hin_off);
  a.S = at<float>(scratch, lay.s_off);
  a.wt = at<char>(saved_ws, lay.wt_off);
  a.wtb = at<char>(saved_ws, lay.wtb_off);

  bool dispatched = false;
#define SSD_DISPATCH(TT, Q_, P_, N_)                                  \
  if (!dispatched && lay.Q == Q_ && lay.P == P_ && lay.N == N_) {     \
    run_fwd<TT, Q_, P_, N_>(lay, a, stream, probe);                   \
    dispatched = true;                                                \
  }
#define SSD_DISPATCH_BF16(Q_, P_, N_) SSD_DISPATCH(bf16, Q_, P_, N_)
#define SSD_DISPATCH_F32(Q_, P_, N_) SSD_DISPATCH(float, Q_, P_, N_)
  if (s->dtype == SSD_BF16) { SSD_BF16_CONFIGS(SSD_DISPATCH_BF16) }
  else { SSD_F32_CONFIGS(SSD_DISPATCH_F32) }
  if (!dispatched) return SSD_ERR_UNSUPPORTED;
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
  const Layout lay = make_layout(s);
  if (!sv->saved_ws || sv->saved_ws_bytes < lay.saved_bytes) return SSD_ERR_WORKSPACE;
  if (!scratch || scratch_bytes < lay.bwd_bytes) return SSD_ERR_WORKSPACE;

  BwdArgs a{};
  a.x = sv->x; a.dt = sv->dt; a.B = sv->B; a.C = sv->C; a.dy = dy; a.A = sv->A; a.D = sv->D;
  a.cs = at<float>(sv->saved_ws, lay.cs_off);
  a.hin = at<char>(sv->saved_ws, lay.hin_off);
  a.w = at<char>(sv->saved_ws, lay.wtb_off);
  a.dx = dx; a.ddt = ddt; a.dB = dB; a.dC = dC; a.dA = dA; a.dD = dD;
  a.dfinal = dfinal_state; a.dinit = dinitial_state;
  a.dhloc = at<float>(scratch, lay.dhloc_off);
  a.gst = at<char>(scratch, lay.g_off);
  a.dw = at<float>(scratch, lay.dw_off);
  a.dcpart = at<float>(scratch, lay.dcpart_off);
  a.dbpart = at<float>(scratch, lay.dbpart_off);
  a.dapart = at<float>(scratch, lay.dapart_off);
  a.ddpart = at<float>(scratch, lay.ddpart_off);
  a.dlpart = at<float>(scratch, lay.dlpart_off);
  a.dlscal = at<float>(scratch, lay.dlscal_off);

  bool dispatched = false;
#define SSD_DISPATCH_B(TT, Q_, P_, N_)                                \
  if (!dispatched && lay.Q == Q_ && lay.P == P_ && lay.N == N_) {     \
    run_bwd<TT, Q_, P_, N_>(lay, a, stream, probe);                   \
    dispatched = true;                                                \
  }
#define SSD_DISPATCH_B_BF16(Q_, P_, N_) SSD_DISPATCH_B(bf16, Q_, P_, N_)
#define SSD_DISPATCH_B_F32(Q_, P_, N_) SSD_DISPATCH_B(float, Q_, P_, N_)
  if (s->dtype == SSD_BF16) { SSD_BF16_CONFIGS(SSD_DISPATCH_B_BF16) }
  else { SSD_F32_CONFIGS(SSD_DISPATCH_B_F32) }
  if (!dispatched) return SSD_ERR_UNSUPPORTED;
  if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
  return SSD_OK;
}

}  // extern "C"
