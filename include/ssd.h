/*
 * libssd -- Mamba-2 selective state-space (SSD) chunked scan, forward and
 * backward, for AMD Instinct MI355X (gfx950).
 *
 * The operation is the Mamba-2 layer's state-space recurrence, the kernel that
 * the Zyphra/AMD post "Training Transformers and Hybrid models on AMD Instinct
 * MI300X Accelerators" (section "Mamba-2") writes forward and backward GPU
 * kernels for.  The post gives no formula; the layer it names computes, for
 * every batch b and head h (group g = h / (nheads / ngroups)):
 *
 *     S_{-1} = S0 (initial state, zero unless given)    state, dstate x headdim
 *     S_t    = exp(dt_t A_h) S_{t-1} + dt_t B_t x_t^T
 *     y_t    = S_t^T C_t + D_h x_t
 *     final_state = S_{L-1}
 *
 * with a scalar A_h and D_h per head.  ssd_bwd returns the exact reverse-mode
 * gradients of the scalar sum_t <dy_t, y_t> + <dS_fin, final_state> (dS_fin,
 * the final-state cotangent, zero unless given): dx, ddt, dA, dB, dC, dD and,
 * on request, dS0.  A nonzero initial state and cotangent are what carry a
 * sequence across calls: a sequence cut in two runs as two calls, the second
 * started from the first's final_state, and the second's dS0 is the first's
 * dS_fin in the backward.
 *
 * Preconditions (not checked on the device): A_h <= 0 and dt >= 0, so every
 * per-step decay lies in [0, 1]; dt is the step after any softplus.
 *
 * Layouts (dense, row-major, element strides implied by the shape):
 *     x, y, dx, dy     [batch][seqlen][nheads][headdim]    dtype
 *     dt, ddt          [batch][seqlen][nheads]             dtype
 *     B, C, dB, dC     [batch][seqlen][ngroups][dstate]    dtype
 *     A, D, dA, dD     [nheads]                            float32
 *     final_state, initial_state, dfinal_state, dinitial_state
 *                      [batch][nheads][headdim][dstate]    float32
 *                      (element [p][n] is the state's entry [n][p])
 * "dtype" is float32 (SSD_F32) or bfloat16 (SSD_BF16); accumulation is
 * always float32.  SSD_FP8: x, B and C are OCP FP8 E4M3 codes (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits; one byte each, no scale) in
 * both passes, every other dtype tensor (dt, y, dy, dx, ddt, dB, dC)
 * bfloat16; every product widens the codes to bfloat16 exactly (the
 * forward's C.B^T runs on the FP8 matrix cores where a launch of its own
 * forms it).  Every pointer is a device pointer aligned
 * to 16 bytes.
 *
 * Ownership: the caller allocates every buffer (inputs, outputs, the saved
 * workspace and the scratch workspaces); the library never allocates or frees
 * device memory and keeps no global mutable state, so calls are reentrant.
 * The one exception is ssd_fwd_noalloc, whose scratch is a static device
 * buffer of the library (one per GPU) and whose calls on one GPU must not
 * overlap.  All work is enqueued on `stream`; the calls return without
 * synchronising.
 *
 * Errors: argument checks run on the host before anything is enqueued; on
 * failure nothing is launched and an error code is returned.  A HIP launch
 * error after the checks is reported as SSD_ERR_HIP.  No C++ exception
 * crosses this interface.
 */
#ifndef LIBSSD_SSD_H
#define LIBSSD_SSD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSD_OK = 0,
    SSD_ERR_INVALID_ARGUMENT = 1, /* null pointer, non-positive size, nheads % ngroups, unknown flag, misalignment */
    SSD_ERR_UNSUPPORTED = 2,      /* (dtype, chunk, headdim, dstate) combination not compiled in */
    SSD_ERR_WORKSPACE = 3,        /* workspace pointer null or smaller than the *_bytes query */
    SSD_ERR_HIP = 4,              /* a HIP call or kernel launch failed */
    SSD_ERR_TOO_LARGE = 5         /* ssd_fwd_noalloc: forward scratch needed > SSD_FWD_STATIC_SCRATCH_BYTES */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1, SSD_FP8 = 2 } ssd_dtype;

/* ssd_shape.flags.  SSD_DT_SOFTPLUS: the dt argument is the raw step and the
 * scan uses dt_t = softplus(dt_raw_t + dt_bias_h), softplus(z) = log(1 + e^z)
 * (z itself for z > 20), the Mamba-2 block's step parameterisation; in bf16
 * mode that step is rounded to bfloat16 once.  ddt is then the gradient of
 * the raw step, ddt_raw = ddt_step * sigmoid(dt_raw + dt_bias), and ssd_bwd
 * can return the bias gradient, the sum of ddt_raw over batch and tokens. */
enum { SSD_DT_SOFTPLUS = 1 };

/* Problem size.  chunk is the chunk length Q of the chunked scan; when
 * seqlen is not a multiple of it, the last chunk of every sequence holds the
 * remaining seqlen mod Q tokens.  dtype is an ssd_dtype.  Compiled (chunk, headdim,
 * dstate) combinations (others give SSD_ERR_UNSUPPORTED):
 *   SSD_BF16, SSD_FP8: chunk 128 or 256 with (headdim, dstate) (16, 16), (64, 64), (64, 128)
 *   SSD_F32 : chunk 64, 128 or 256 with (16, 16); chunk 64 or 128 with (64, 64);
 *             chunk 64 with (64, 128)                                          */
typedef struct {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
    int32_t dtype;
    int32_t flags;    /* 0 or SSD_DT_SOFTPLUS */
} ssd_shape;

/* Forward-to-backward context, filled by ssd_fwd.  It borrows the input
 * pointers (not initial_state) and the saved workspace: x, dt, A, B, C, D and saved_ws must stay
 * alive and unmodified until the ssd_bwd that consumes this context has
 * finished on its stream. */
typedef struct {
    ssd_shape shape;
    const void *x, *dt, *B, *C;
    const float *A, *D;
    const void *saved_ws;
    size_t saved_ws_bytes;
} ssd_saved;

/* Kernel identifiers, for timing one kernel with an ssd_probe. */
typedef enum {
    SSD_K_CUMSUM_BMM = 0,        /* one launch: per-chunk inclusive cumsum of dt*A, and C.B^T per chunk and
                                    group for the forward chunk kernel */
    SSD_K_CHUNK_STATE = 1,       /* decay-weighted B^T x per chunk and head */
    SSD_K_STATE_PASSING = 2,     /* sequential inter-chunk state scan */
    SSD_K_CHUNK_SCAN = 3,        /* intra-chunk masked product + state-to-output + D x */
    SSD_K_CHUNK_STATE_BWD = 4,   /* exp(cs) C^T dy per chunk and head */
    SSD_K_STATE_PASSING_BWD = 5, /* reverse inter-chunk state scan */
    SSD_K_CHUNK_SCAN_BWD = 6,    /* dx, ddt and per-chunk dA/dD partials (chunk kernel, which forms C.B^T
                                    again in fp32, + dl assembly) */
    SSD_K_DW_HEADS = 7,          /* one launch of the group-level head sums: masked dY.X^T (dW) and the
                                    dC / dB state terms, per chunk, group and head slice */
    SSD_K_BC_FINAL = 8,          /* dC and dB in one launch: slice sums + dW.B and dW^T.C */
    SSD_K_DA_DD = 9,             /* fixed-order dA / dD reduction */
    SSD_NUM_KERNELS = 10
} ssd_kernel_id;

/* Optional timing hook: when passed to ssd_fwd/ssd_bwd and `kernel` names a
 * kernel that call launches, `start` is recorded on the stream right before
 * that launch and `stop` right after it.  Both events are created by the
 * caller (hipEventCreate).  Pass NULL for no timing. */
typedef struct {
    int32_t kernel;
    int32_t reserved;
    hipEvent_t start;
    hipEvent_t stop;
} ssd_probe;

/* Workspace sizes in bytes for a shape; 0 if the shape is invalid or
 * unsupported.  saved: kept from ssd_fwd to ssd_bwd (per-chunk cumsums and
 * the chunk-entry states).  fwd/bwd scratch: only used during the call. */
size_t ssd_saved_bytes(const ssd_shape *shape);
size_t ssd_fwd_scratch_bytes(const ssd_shape *shape);
size_t ssd_bwd_scratch_bytes(const ssd_shape *shape);

/* Where the chunked algorithm's intermediates sit, as byte offsets into the
 * workspace each field names, so that they can be inspected and checked one
 * kernel at a time (Mamba-2 SSD chunked algorithm: the in-chunk cumsum, the
 * chunk states, state passing; and the reverse of each in the backward).
 * With K = ceil(seqlen / chunk) chunks of Q = chunk rows, the last one
 * zero-padded when Q does not divide seqlen, and "state" meaning float32
 * for SSD_F32 and bf16 otherwise (SSD_FP8 included):
 *   in saved_ws, written by ssd_fwd:
 *     cs          float32 [b][H][K][Q]  sum_{j <= i} dt_j A_h within chunk k
 *     step        float32 [b][H][K][Q]  the dt the scan used (softplus(dt + dt_bias)
 *                                       with SSD_DT_SOFTPLUS; 0 on padded rows)
 *     hin         state [b][K][H][P][N]  the state entering chunk k
 *   in the forward scratch, written by ssd_fwd:
 *     chunk_state state [b][K][H][P][N]  chunk k's contribution from a zero state:
 *                                       sum_i exp(cs_{Q-1} - cs_i) dt_i x_i B_i^T
 *   in the backward scratch, written by ssd_bwd:
 *     dhloc       state [b][K][H][P][N]  sum_i exp(cs_i) dy_i C_i^T over chunk k
 *     gstate      state [b][K][H][P][N]  the gradient with respect to the state
 *                                       leaving chunk k
 * The values stay until the workspace is next written; the library never
 * reads them back from the caller except through ssd_bwd's saved context.
 * Returns the ssd_check_shape error for an invalid or unsupported shape, and
 * SSD_ERR_INVALID_ARGUMENT for a NULL pointer; *out is written on SSD_OK only. */
typedef struct {
    size_t cs, step, hin;
    size_t chunk_state;
    size_t dhloc, gstate;
} ssd_regions;
ssd_status ssd_workspace_regions(const ssd_shape *shape, ssd_regions *out);

/* SSD_OK if the shape is valid and its (dtype, chunk, headdim, dstate) is
 * compiled in; otherwise the error ssd_fwd would return for it. */
ssd_status ssd_check_shape(const ssd_shape *shape);

/* Forward pass: y and final_state from x, dt, A, B, C, D, starting from
 * initial_state (NULL means zero; it is read during the call only, the
 * backward keeps its own copy in saved_ws).  dt_bias [nheads] float32 is
 * read only with SSD_DT_SOFTPLUS (NULL means zero).
 * y is written; final_state is written if non-NULL.  saved_ws (>=
 * ssd_saved_bytes) receives what ssd_bwd needs; saved_out, if non-NULL, is
 * filled with the context ssd_bwd consumes.  scratch (>= ssd_fwd_scratch_bytes)
 * is free to reuse once the call's work has finished on the stream.
 * probe may be NULL. */
ssd_status ssd_fwd(const ssd_shape *shape,
                   const void *x, const void *dt, const float *A,
                   const void *B, const void *C, const float *D,
                   const float *dt_bias, const float *initial_state,
                   void *y, float *final_state,
                   void *saved_ws, size_t saved_ws_bytes, ssd_saved *saved_out,
                   void *scratch, size_t scratch_bytes,
                   hipStream_t stream, const ssd_probe *probe);

/* Forward pass that allocates nothing and takes no scratch argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments,
 * results and saved context as ssd_fwd (the saved workspace is still the
 * caller's); its scratch is a static device buffer of the library, 96 MiB
 * per GPU (SSD_FWD_STATIC_SCRATCH_BYTES), held from the library's load on a
 * GPU until the process ends.  Problems whose ssd_fwd_scratch_bytes exceeds
 * it return SSD_ERR_TOO_LARGE before anything is launched (the Mamba2-2.7B
 * shape, 4 x 4096 tokens with 80 heads of 64 x 128 in bf16, needs 80 MiB).
 * `stream` must belong to the current device (SSD_ERR_INVALID_ARGUMENT
 * otherwise; the null stream always does).  Every call on one GPU shares
 * that GPU's buffer, so calls that overlap on one GPU (on different streams,
 * or from different threads without ordering) race; calls ordered on one
 * stream do not.  Nothing in the buffer needs to start at zero. */
#define SSD_FWD_STATIC_SCRATCH_BYTES (96u * 1024u * 1024u)
ssd_status ssd_fwd_noalloc(const ssd_shape *shape,
                           const void *x, const void *dt, const float *A,
                           const void *B, const void *C, const float *D,
                           const float *dt_bias, const float *initial_state,
                           void *y, float *final_state,
                           void *saved_ws, size_t saved_ws_bytes, ssd_saved *saved_out,
                           hipStream_t stream, const ssd_probe *probe);

/* Backward pass: gradients of sum <dy, y> + <dfinal_state, final_state>
 * for the forward that filled `saved` (dfinal_state NULL means zero).
 * dx, ddt, dA, dB, dC, dD are overwritten (not accumulated); dinitial_state,
 * the gradient of the forward's initial state, is written if non-NULL (also
 * when the forward started from zero); ddt_bias [nheads] float32, the dt_bias
 * gradient, is written if non-NULL and the shape has SSD_DT_SOFTPLUS.
 * scratch must hold ssd_bwd_scratch_bytes(&saved->shape). probe may be NULL. */
ssd_status ssd_bwd(const ssd_saved *saved, const void *dy, const float *dfinal_state,
                   void *dx, void *ddt, float *dA, void *dB, void *dC, float *dD,
                   float *ddt_bias, float *dinitial_state,
                   void *scratch, size_t scratch_bytes,
                   hipStream_t stream, const ssd_probe *probe);

/* ---- Causal depthwise conv1d ------------------------------------------
 *
 * The convolution that feeds the scan in a Mamba block (the "causal conv"
 * kernel the LightOn page "Training Mamba Models on AMD MI250/MI250X GPUs
 * with Custom Kernels", section "Individual Kernels", times): per channel c, a width-W filter w[c][0..W-1], a bias and
 * an optional SiLU,
 *     z[b][t][c] = bias[c] + sum_k w[c][k] x[b][t - (W-1) + k][c],
 *     y = silu(z) = z / (1 + e^-z)   (or y = z)
 * Rows before the sequence are x_prev's [b][W-1][C] (times -(W-1)..-1) or
 * zero: with x_prev a sequence cut into pieces runs as separate calls.
 * ssd_conv1d_bwd returns the gradients of <dy, y>: dx, dw, dbias and the
 * halo's gradient dx_prev (the last W-1 rows of the previous piece add it).
 *
 * Layouts: x, y, dy, dx [batch][seqlen][channels] and x_prev, dx_prev
 * [batch][width-1][channels] in `dtype`; w, dw [channels][width] and bias,
 * dbias [channels] float32.  Device pointers, 16-byte aligned; bias, x_prev,
 * dbias and dx_prev may be NULL (absent).  Supported: width 2..4, channels a
 * multiple of 4 (else SSD_ERR_UNSUPPORTED).  Same ownership, stream and error
 * rules as ssd_fwd / ssd_bwd; dw and dbias are overwritten, fixed-order sums
 * (no atomics). */
typedef struct {
    int64_t batch, seqlen, channels;
    int32_t width;
    int32_t dtype;     /* ssd_dtype of x, x_prev, y, dy, dx, dx_prev */
    int32_t silu;      /* 1: y = silu(z); 0: y = z */
    int32_t reserved;  /* must be 0 */
} ssd_conv_shape;

ssd_status ssd_conv1d_check_shape(const ssd_conv_shape *shape);
size_t ssd_conv1d_bwd_scratch_bytes(const ssd_conv_shape *shape);
ssd_status ssd_conv1d_fwd(const ssd_conv_shape *shape, const void *x, const float *w, const float *bias,
                          const void *x_prev, void *y, hipStream_t stream);
ssd_status ssd_conv1d_bwd(const ssd_conv_shape *shape, const void *x, const float *w, const float *bias,
                          const void *x_prev, const void *dy, void *dx, float *dw, float *dbias, void *dx_prev,
                          void *scratch, size_t scratch_bytes, hipStream_t stream);

/* Static description of a status code (an ssd_status value; any other
 * value gives "unknown status"). */
const char *ssd_status_string(int32_t status);

/* Static name of a kernel id (NULL if out of range). */
const char *ssd_kernel_name(int32_t kernel);

/* Library version, "major.minor.patch". */
const char *ssd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBSSD_SSD_H */
