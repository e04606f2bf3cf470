/*
 * ssmbwd.h — C ABI of the MI355X (gfx950) selective-scan backward library.
 *
 * Operations are those of the Mamba layer backward walked by mamba-rs 0.5.1
 * (src/mamba_ssm/cpu/backward.rs, backward_mamba_layer_batched, and the
 * backbone around it, backward_mamba_backbone_batched), with the closed-form
 * RMSNorm and cumsum backward of rlx-cpu 0.2.17 (src/training_bwd.rs,
 * rms_norm_backward_row, cumsum_backward_row).  The CPU pages run them as
 * sequential loops over one sequence; here every call is a batch of sequences
 * on one GPU.
 *
 * Conventions for every entry point
 *  - Memory: all tensor pointers are DEVICE pointers to contiguous row-major
 *    storage owned by the caller.  The library never allocates or frees device
 *    memory; scratch space is a caller-provided workspace whose size the
 *    matching *_workspace_size() call returns, at a 256-byte aligned address
 *    (hipMalloc's alignment).  Gradients are overwritten
 *    unless the call's flags include SSM_BWD_ACCUMULATE (ssm_bwd_flags).
 *  - Storage dtype: [batch, seqlen, *] activations and their gradients are
 *    SSM_F32 (float) or SSM_BF16 (bfloat16, round-to-nearest-even on store).
 *    Parameters (A_log, D, conv weight and bias, norm weight) and their
 *    gradients are always float.  Arithmetic is float32 throughout.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *    stream).  Calls are asynchronous on that stream: no host synchronisation,
 *    no hidden allocation.
 *  - Errors: arguments are checked before anything is launched; a bad call
 *    returns a non-zero ssm_status and leaves every output untouched.  A
 *    failed launch returns SSM_ERR_LAUNCH.  ssm_last_error() gives a message
 *    for the calling thread's last failure.
 *  - Results are deterministic: no atomics; every reduction has a fixed order,
 *    so two calls with the same inputs and dims give bitwise equal outputs.
 *  - Thread safety: calls on different streams may run concurrently as long
 *    as they do not share a workspace.
 */
#ifndef SSMBWD_H
#define SSMBWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssm_status {
  SSM_OK = 0,
  SSM_ERR_INVALID_ARG = 1,  /* null pointer, negative size, inconsistent stride */
  SSM_ERR_UNSUPPORTED = 2,  /* e.g. d_state outside {4, 8, 16}, misaligned bf16 rows */
  SSM_ERR_WORKSPACE = 3,    /* workspace pointer null, smaller than required or not 256-byte aligned */
  SSM_ERR_LAUNCH = 4        /* a kernel launch failed */
} ssm_status;

typedef enum ssm_dtype { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

/* Flags of the backward entry points (bitwise or; other bits are rejected).
 * SSM_BWD_ACCUMULATE: parameter gradients (d_A_log, d_D; dW and db of
 * linear_bwd; d_w and d_bias of conv1d_bwd; dw of rmsnorm_bwd) are added into
 * the caller's buffers instead of overwriting them, as mamba-rs's gradient
 * accumulators take `+=` (Phase B3's d_layer.a_log and d_param), so that
 * micro-batches sum into one set of buffers.  Per-element gradients (d_u,
 * d_delta, d_z, d_B, d_C, dX, d_x) are written either way.  Calls on an empty
 * batch then leave the buffers as they are. */
typedef enum ssm_bwd_flags {
  SSM_BWD_SOFTPLUS = 1,      /* ssm_scan_bwd*: the softplus epilogue (see ssm_scan_bwd) */
  SSM_BWD_ACCUMULATE = 2,
  SSM_BWD_ACCUMULATE_DX = 4  /* linear_bwd: dX is added into dX's contents */
} ssm_bwd_flags;

/* Shape of one selective-scan call.
 *   u, delta, z, d_out, d_u, d_delta, d_z : [batch, seqlen, d_inner]
 *   B, C                                   : [batch, seqlen, *] rows of stride ld_bc,
 *                                            the d_state values of step t at row (b*seqlen+t)
 *   d_B, d_C                               : same, row stride ld_dbc
 *   A_log, d_A_log                         : [d_inner, d_state] (index d*d_state + n)
 *   D, d_D                                 : [d_inner]
 * ld_bc / ld_dbc = d_state for standalone tensors; a larger stride lets B and C
 * (and their gradients) live inside the x_proj row [dt | B | C] as the layer
 * keeps them.  For SSM_BF16 the B, C, d_B, d_C base pointers must be 4-byte
 * aligned and the strides even.
 * seg_len: length of the time segments that run in parallel and are joined by
 * the cross-segment carries; 0 picks one from the shape.  Must be 0 or a
 * multiple of 8.  Results do not depend on it beyond float rounding.
 * ld_z: row stride of z and d_z (0 means d_inner), so that the gate and its
 * gradient can be the second half of the in_proj output row [x | z].
 * seqlen * max(d_inner, ld_z) must stay below 2^32. */
typedef struct ssm_dims {
  int32_t batch;
  int32_t seqlen;
  int32_t d_inner;
  int32_t d_state;
  int32_t ld_bc;
  int32_t ld_dbc;
  int32_t seg_len;
  int32_t ld_z;
} ssm_dims;

const char* ssm_status_string(int status);
const char* ssm_last_error(void);

/* ---------------------------------------------------------------------------
 * ssm_scan_bwd — backward of the selective scan with its output gate.
 * mamba-rs cpu/backward.rs, Phase B2 (gating backward) and Phase B3
 * (sequential SSM BPTT), forward as implied by the saved da_exp/h_prev/h_curr:
 *     A = -exp(A_log),  a_t = exp(delta_t A),  h_t = a_t h_{t-1} + delta_t u_t B_t,
 *     h_{-1} = 0,  y_t = C_t . h_t + D u_t,  out_t = y_t * SiLU(z_t).
 * Given d_out = dL/d out it writes dL/du, dL/d delta, dL/d A_log, dL/dB, dL/dC,
 * dL/dD and dL/dz.  The forward states are recomputed in chunks; no per-step
 * state is read from or written to memory by the caller.
 * flags & SSM_BWD_SOFTPLUS: delta is taken to be softplus(raw) (the layer's
 * dt_proj output) and d_delta receives dL/d raw instead, using
 * sigmoid(raw) = 1 - exp(-delta) and passing the gradient through where
 * delta > 20 (the page's "Softplus backward" step, threshold 20).
 * flags & SSM_BWD_ACCUMULATE: d_A_log and d_D are added into.
 * All output pointers are required.  Workspace: ssm_scan_bwd_workspace_size().
 * ------------------------------------------------------------------------- */
size_t ssm_scan_bwd_workspace_size(const ssm_dims* dims, int dtype);
int ssm_scan_bwd(const void* u, const void* delta, const float* A_log, const void* B,
                 const void* C, const float* D, const void* z, const void* d_out,
                 void* d_u, void* d_delta, float* d_A_log, void* d_B, void* d_C,
                 float* d_D, void* d_z, int flags,
                 void* workspace, size_t ws_bytes, const ssm_dims* dims, int dtype,
                 void* stream);

/* Same as ssm_scan_bwd, with stage timing: `stage_events` (nullable) points to
 * 5 hipEvent_t handles (passed as void*, each may be null) created by the
 * caller; event k is recorded on `stream` before stage k+1 / after stage k of
 * the call: [0] start, [1] after the segment summaries, [2] after the carries,
 * [3] after the main backward sweep, [4] after the final reductions.
 * For profiling callers (the bench); results are identical to ssm_scan_bwd. */
int ssm_scan_bwd_timed(const void* u, const void* delta, const float* A_log, const void* B,
                       const void* C, const float* D, const void* z, const void* d_out,
                       void* d_u, void* d_delta, float* d_A_log, void* d_B, void* d_C,
                       float* d_D, void* d_z, int flags,
                       void* workspace, size_t ws_bytes, const ssm_dims* dims, int dtype,
                       void* stream, void* const* stage_events);

/* ---------------------------------------------------------------------------
 * ssm_scan_bwd_ckpt — ssm_scan_bwd for a caller whose forward kept the state
 * before every 8-step chunk, as ssm_scan_fwd writes it with ckpt_every = 8:
 * h_ckpt[b, k, n, d] = h_{8k - 1} (zero for k = 0), k = 0 .. ceil(seqlen / 8) - 1,
 * float, [batch, ceil(seqlen / 8), d_state, d_inner] contiguous, read only.
 * (mamba-rs Phase B3 reads saved per-step states back; here only the chunk
 * boundaries are kept.)  The backward then skips rebuilding the states of each
 * segment: its first pass only sums delta and the adjoint summary of each
 * segment, and each chunk starts from the given state.  Same outputs as
 * ssm_scan_bwd up to float rounding when h_ckpt holds the forward's states;
 * arguments otherwise as ssm_scan_bwd, with `stage_events` as in
 * ssm_scan_bwd_timed (nullable).  h_ckpt must not be null.
 * Workspace: ssm_scan_bwd_ckpt_workspace_size() (smaller: no local
 * checkpoints).
 * ------------------------------------------------------------------------- */
size_t ssm_scan_bwd_ckpt_workspace_size(const ssm_dims* dims, int dtype);
int ssm_scan_bwd_ckpt(const void* u, const void* delta, const float* A_log, const void* B,
                      const void* C, const float* D, const void* z, const void* d_out,
                      const float* h_ckpt, void* d_u, void* d_delta, float* d_A_log, void* d_B,
                      void* d_C, float* d_D, void* d_z, int flags,
                      void* workspace, size_t ws_bytes, const ssm_dims* dims, int dtype,
                      void* stream, void* const* stage_events);

/* ---------------------------------------------------------------------------
 * ssm_scan_bwd_ckpt_noalloc — ssm_scan_bwd_ckpt without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving or training loops, harnesses that forbid hipMalloc.
 * Same kernels, arguments and outputs as ssm_scan_bwd_ckpt (no stage events).
 * Its scratch is a static device array of ssm_scan_bwd_ckpt_noalloc_capacity()
 * bytes (64 MiB), one copy per GPU that runs the call, held from the first
 * call on that GPU until the process ends.  A shape whose
 * ssm_scan_bwd_ckpt_workspace_size() exceeds it is rejected with
 * SSM_ERR_WORKSPACE before anything is launched (the mamba-370m shape, batch 8,
 * seqlen 2048, d_inner 2048, d_state 16, needs about 35 MB).
 * The call itself allocates nothing: on its first call on a device it looks up
 * the array's device address (hipGetSymbolAddress) and keeps it.  `stream`
 * must belong to the current device (SSM_ERR_INVALID_ARG otherwise).
 * Every call on one GPU shares that GPU's scratch and leaves its contents
 * behind (nothing in it needs to start at zero): two calls whose executions
 * overlap on one GPU, on different streams or from different threads, race
 * and give wrong results.  Serialise them on one stream.
 * ------------------------------------------------------------------------- */
size_t ssm_scan_bwd_ckpt_noalloc_capacity(void);
int ssm_scan_bwd_ckpt_noalloc(const void* u, const void* delta, const float* A_log, const void* B,
                              const void* C, const float* D, const void* z, const void* d_out,
                              const float* h_ckpt, void* d_u, void* d_delta, float* d_A_log,
                              void* d_B, void* d_C, float* d_D, void* d_z, int flags,
                              const ssm_dims* dims, int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * ssm_scan_fwd —the forward recurrence above (the page's forward is implied
 * by the states Phase B3 reads back).  Writes y (nullable), out = y * SiLU(z)
 * (nullable; requires z) and, if h_ckpt is not null, the state before every
 * ckpt_every-th step: h_ckpt[b, k, n, d] = h_{k*ckpt_every - 1} (zero for k = 0),
 * k = 0 .. ceil(seqlen / ckpt_every) - 1, float.  ckpt_every must be a multiple
 * of 8 when h_ckpt is given.  Workspace: ssm_scan_fwd_workspace_size().
 * ------------------------------------------------------------------------- */
size_t ssm_scan_fwd_workspace_size(const ssm_dims* dims, int dtype);
int ssm_scan_fwd(const void* u, const void* delta, const float* A_log, const void* B,
                 const void* C, const float* D, const void* z, void* y, void* out,
                 float* h_ckpt, int ckpt_every, void* workspace, size_t ws_bytes,
                 const ssm_dims* dims, int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * gating_bwd — Phase B2 on its own: gated = y * SiLU(z);
 *     d_y = d_out * SiLU(z),  d_z = d_out * y * s * (1 + z (1 - s)),  s = sigmoid(z).
 * All five tensors hold n elements of the same dtype.  No workspace.
 * ------------------------------------------------------------------------- */
int gating_bwd(const void* d_out, const void* y, const void* z, void* d_y, void* d_z,
               int64_t n, int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * conv1d_bwd — Phase B6: SiLU backward on the conv output, then the causal
 * depthwise conv backward (the page's reverse loop with a shift-register
 * carry, computed here as a stencil).  Forward (recomputed here):
 *     c[b,t,d] = bias[d] + sum_k w[d,k] x[b, t-(d_conv-1)+k, d]   (zero before t = 0),
 *     u = SiLU(c).
 * d_u is dL/du.  Writes d_x[b,t,d] = sum_k g[b, t+(d_conv-1)-k, d] w[d,k] with
 * g = d_u * SiLU'(c), d_w[d,k] = sum_{b,t} g[b,t,d] x[b,t-(d_conv-1)+k,d] and
 * d_bias[d] = sum g.  x, d_u, d_x rows have strides ld_x, ld_du, ld_dx (>= d_inner)
 * so that x can be the first half of the in_proj output row and d_x the first
 * half of its gradient.  w [d_inner, d_conv] and bias are float; d_conv <= 8.
 * flags: 0 or SSM_BWD_ACCUMULATE (d_w and d_bias added into).
 * Workspace: conv1d_bwd_workspace_size().
 * ------------------------------------------------------------------------- */
size_t conv1d_bwd_workspace_size(int batch, int seqlen, int d_inner, int d_conv);
int conv1d_bwd(const void* x, const float* w, const float* bias, const void* d_u,
               void* d_x, float* d_w, float* d_bias, int batch, int seqlen, int d_inner,
               int d_conv, int ld_x, int ld_du, int ld_dx, int flags, void* workspace,
               size_t ws_bytes, int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * reverse_linear_scan — the one-state adjoint sweep of mamba-rs cpu/backward.rs
 * Phase B3 (d_h <- da * d_h after each step) as a primitive, along t of
 * time-major [batch, seqlen, channels] tensors (contiguous, channel fastest):
 *     x_t = b_t + a_{t+1} x_{t+1},   x_seqlen = 0         (exclusive == 0)
 *     x_t = a_{t+1} (b_{t+1} + ...) = (inclusive x)_t - b_t  (exclusive != 0)
 * a == NULL means a = 1: the cumsum backward of rlx-cpu training_bwd.rs
 * cumsum_backward_row (suffix sums, inclusive or exclusive) along t for every
 * (batch, channel).  a, b, x share dtype (SSM_F32 / SSM_BF16 storage, float
 * arithmetic); x must not overlap a or b.  Workspace:
 * reverse_linear_scan_workspace_size(batch, seqlen, channels, a != NULL)
 * (0 bytes for short sequences; the workspace pointer may then be null).
 * Limits: batch <= 65535 and batch * channels < 2^31, else SSM_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------- */
size_t reverse_linear_scan_workspace_size(int batch, int seqlen, int channels, int has_a);
int reverse_linear_scan(const void* a, const void* b, void* x, int batch, int seqlen, int channels,
                        int exclusive, void* workspace, size_t ws_bytes, int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * rmsnorm_bwd — rlx-cpu training_bwd.rs rms_norm_backward_row over `rows`
 * rows of `dim`, without the shift term (Phase B8 of the layer passes only the
 * norm weight), plus the residual of Phase B8:
 *     inv_r = 1/sqrt(mean(x^2) + eps)
 *     dx = inv_r w dy - inv_r^3 x mean(dy w x)  (+ d_residual if not null)
 *     dw = sum over rows of dy x inv_r
 * x, dy, d_residual, dx: [rows, dim] in dtype; w, dw: [dim] float.
 * flags: 0 or SSM_BWD_ACCUMULATE (dw added into).
 * Workspace: rmsnorm_bwd_workspace_size().
 * ------------------------------------------------------------------------- */
size_t rmsnorm_bwd_workspace_size(int64_t rows, int dim);
int rmsnorm_bwd(const void* x, const float* w, const void* dy, const void* d_residual,
                void* dx, float* dw, int64_t rows, int dim, float eps, int flags,
                void* workspace, size_t ws_bytes, int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * linear_bwd — the weight-layer backward that mamba-rs cpu/backward.rs runs
 * (sgemm_backward) in Phases B1 (out_proj), B4 (dt_proj, with bias), B5
 * (x_proj) and B7 (in_proj), for Y = X W^T (+ b) with W [N, K] (out, in):
 *     dX = dY W            [M, K]   (bf16; added to dX's contents with SSM_BWD_ACCUMULATE_DX)
 *     dW = dY^T X          [N, K]   (float; added into with SSM_BWD_ACCUMULATE)
 *     db = sum over rows of dY [N] (float; added into with SSM_BWD_ACCUMULATE)
 * flags: SSM_BWD_ACCUMULATE_DX | SSM_BWD_ACCUMULATE or 0.
 * X [M, K] rows of stride ldx, dY [M, N] rows of stride lddy, dX rows of
 * stride lddx, W contiguous; all bf16 (dtype must be SSM_BF16), products on the
 * matrix cores with float accumulation.  dX, dW, db are each nullable (skipped);
 * X may be null when dW is.  X, W, dY need 16-byte aligned bases and row strides
 * that are multiples of 8.  Workspace: linear_bwd_workspace_size() (split-k
 * partial sums; 0 bytes when no split is used).
 * Repeatability: a call repeated with the same shapes and the same set of
 * requested outputs gives the same bits.  When dX and dW are both requested the
 * two products share one launch and dW's split over M is chosen for the pair, so
 * dW may then differ from a dW-only call by float rounding; dX never does.
 * ------------------------------------------------------------------------- */
size_t linear_bwd_workspace_size(int64_t M, int K, int N);
int linear_bwd(const void* X, int64_t ldx, const void* W, const void* dY, int64_t lddy,
               void* dX, int64_t lddx, int flags, float* dW, float* db,
               int64_t M, int K, int N, void* workspace, size_t ws_bytes, int dtype,
               void* stream);

/* linear_fwd — Y[M, N] = X[M, K] W[N, K]^T in bf16 with float accumulation (the
 * forward products whose backward linear_bwd computes; used to build a layer's
 * saved activations).  bias must be null.  Same alignment rules as linear_bwd.
 * Workspace: linear_fwd_workspace_size(). */
size_t linear_fwd_workspace_size(int64_t M, int K, int N);
int linear_fwd(const void* X, int64_t ldx, const void* W, const float* bias, void* Y,
               int64_t ldy, int64_t M, int K, int N, void* workspace, size_t ws_bytes,
               int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * The whole Mamba layer around the scan, as mamba-rs cpu/backward.rs
 * backward_mamba_layer_batched walks it (Phases B1-B8); its forward is read
 * back from those phases:
 *     xn    = RMSNorm(x; norm_w, eps)                          (B8)
 *     xz    = xn W_in^T,  x_b = xz[:, :d_inner], z = xz[:, d_inner:]   (B7)
 *     u     = SiLU(causal depthwise conv(x_b; conv_w, conv_b))  (B6)
 *     xdbl  = u W_x^T = [dt_in | B | C]  (dt_rank, d_state, d_state columns)  (B5, B3)
 *     delta = softplus(dt_in W_dt^T + b_dt), passed through above 20        (B4, B3)
 *     y     = selective scan(u, delta, A_log, B, C, D)          (B3)
 *     out   = (y * SiLU(z)) W_out^T + x                         (B2, B1, B8 residual)
 * Activations [batch, seqlen, *] are bf16 (rows of their own width, no padding);
 * weight matrices are bf16 [out, in]; norm_w, conv_w [d_inner, d_conv], conv_b,
 * b_dt, A_log [d_inner, d_state], D and every parameter gradient are float.
 * d_model, d_inner, dt_rank and dt_rank + 2 d_state must be multiples of 8,
 * d_state in {4, 8, 16}, d_conv <= 8, d_model <= 4096, all pointers 16-byte aligned.
 * ------------------------------------------------------------------------- */
typedef struct ssm_layer_dims {
  int32_t batch;
  int32_t seqlen;
  int32_t d_model;
  int32_t d_inner;
  int32_t d_state;
  int32_t dt_rank;
  int32_t d_conv;
  int32_t seg_len; /* the scan's segment length, 0 = auto (see ssm_dims) */
  float eps;       /* RMSNorm epsilon */
} ssm_layer_dims;

typedef struct ssm_layer_weights {
  const float* norm_w; /* [d_model] */
  const void* W_in;    /* [2 d_inner, d_model] */
  const float* conv_w; /* [d_inner, d_conv] */
  const float* conv_b; /* [d_inner] */
  const void* W_x;     /* [dt_rank + 2 d_state, d_inner] */
  const void* W_dt;    /* [d_inner, dt_rank] */
  const float* b_dt;   /* [d_inner] */
  const float* A_log;  /* [d_inner, d_state] */
  const float* D;      /* [d_inner] */
  const void* W_out;   /* [d_model, d_inner] */
} ssm_layer_weights;

/* what the forward keeps for the backward (everything else is recomputed).
 * The last three, the inputs of the out_proj, x_proj and in_proj products, are
 * the activations mamba-rs's MambaLayerFlat keeps as gated, u and post_norm
 * (cpu/backward.rs, backward_mamba_layer_batched, Phases B1, B5 and B7 read
 * them); each is nullable: when given, the forward writes it and the backward
 * reads it instead of recomputing it (the gate, the conv + SiLU and the
 * RMSNorm forward), at 2 bytes per element of extra activation memory. */
typedef struct ssm_layer_saved {
  void* xz;    /* [batch, seqlen, 2 d_inner] in_proj output */
  void* xdbl;  /* [batch, seqlen, dt_rank + 2 d_state] x_proj output */
  void* delta; /* [batch, seqlen, d_inner] softplus output */
  void* y;     /* [batch, seqlen, d_inner] scan output before the gate; may be
                  null when gated is given (only the gate recompute reads it) */
  float* h_ckpt; /* nullable: [batch, ceil(seqlen / 8), d_state, d_inner] float, the
                    scan's state before every 8-step chunk; when given, the forward
                    writes it and the backward starts its scan chunks from it
                    (ssm_scan_bwd_ckpt) instead of rebuilding the states */
  void* gated; /* nullable: [batch, seqlen, d_inner] y * SiLU(z), out_proj's input */
  void* u;     /* nullable: [batch, seqlen, d_inner] SiLU(conv(x_b)), x_proj's and the scan's input */
  void* xn;    /* nullable: [batch, seqlen, d_model] RMSNorm(x), in_proj's input */
} ssm_layer_saved;

typedef struct ssm_layer_grads {
  float* d_norm_w;
  float* d_W_in;
  float* d_conv_w;
  float* d_conv_b;
  float* d_W_x;
  float* d_W_dt;
  float* d_b_dt;
  float* d_A_log;
  float* d_D;
  float* d_W_out;
  int32_t accumulate; /* nonzero: every parameter gradient above is added into
                         (SSM_BWD_ACCUMULATE); d_x is written either way */
} ssm_layer_grads;

/* mamba_layer_fwd — out [batch, seqlen, d_model] and the saved activations
 * (every non-null buffer of `saved` is written).  Workspace:
 * mamba_layer_fwd_workspace_size(). */
size_t mamba_layer_fwd_workspace_size(const ssm_layer_dims* dims);
int mamba_layer_fwd(const void* x, const ssm_layer_weights* w, void* out, const ssm_layer_saved* saved,
                    void* workspace, size_t ws_bytes, const ssm_layer_dims* dims, void* stream);

/* mamba_layer_bwd — Phases B1-B8: from x, the saved activations and
 * d_out = dL/d out, writes d_x = dL/dx (bf16, including the residual path) and
 * every parameter gradient (float; overwritten, or added into when
 * grads->accumulate is set, to sum micro-batches).  Recomputes RMSNorm, the conv
 * + SiLU output and the gate unless `saved` holds them (xn, u, gated), and the
 * scan states unless it holds h_ckpt.  Workspace:
 * mamba_layer_bwd_workspace_size().
 * mamba_layer_bwd_timed: same, recording caller-created hipEvent_t handles
 * (11, each nullable) around its ten stages: [0] start, then after the gate
 * recompute, out_proj, conv recompute, scan, dt_proj, x_proj, conv, RMSNorm
 * recompute, in_proj and RMSNorm backward (a recompute that `saved` makes
 * unnecessary is an empty stage). */
size_t mamba_layer_bwd_workspace_size(const ssm_layer_dims* dims);
int mamba_layer_bwd(const void* x, const ssm_layer_weights* w, const ssm_layer_saved* saved,
                    const void* d_out, void* d_x, const ssm_layer_grads* grads, void* workspace,
                    size_t ws_bytes, const ssm_layer_dims* dims, void* stream);
int mamba_layer_bwd_timed(const void* x, const ssm_layer_weights* w, const ssm_layer_saved* saved,
                          const void* d_out, void* d_x, const ssm_layer_grads* grads, void* workspace,
                          size_t ws_bytes, const ssm_layer_dims* dims, void* stream,
                          void* const* stage_events);

/* ---------------------------------------------------------------------------
 * The backbone around the layers: mamba-rs cpu/backward.rs,
 * backward_mamba_backbone_batched, and the forward it implies:
 *     x_0 = inp W_ip^T + b_ip           (input projection, bias)
 *     x_{l+1} = layer_l(x_l)            (mamba_layer_fwd, l = 0 .. n_layers-1)
 *     out = RMSNorm(x_L; norm_f_w)      (eps = dims->layer.eps, no shift)
 * The backward runs the norm_f backward first, then every layer's backward in
 * reverse order (each hands its d_x to the layer before it), then the input
 * projection's backward (weight and bias; the input gradient d_inp is written
 * only if d_inp is not null: the page discards it).
 * inp [batch, seqlen, input_dim] and W_ip [d_model, input_dim] are bf16 (input_dim
 * a multiple of 8); b_ip (nullable in the forward), norm_f_w and their gradients
 * are float.  `layers`, `saved`, `grads`: arrays of n_layers structs as for
 * mamba_layer_*; `xs`: n_layers + 1 pointers to [batch, seqlen, d_model] bf16
 * buffers, xs[0] the input projection's output, xs[l + 1] layer l's output
 * (xs[n_layers] is norm_f's input).  The forward writes xs, saved and out; the
 * backward reads them (the activations a training step keeps: per layer its
 * input and the four saved tensors, about 0.46 GB per layer of the full layer
 * shape, see ssm_backbone_dims.keep).
 * flags: 0 or SSM_BWD_ACCUMULATE (every parameter gradient of the backbone and
 * of every layer is added into).  Workspaces: the *_workspace_size() calls
 * (one layer's workspace, shared by all layers in turn, plus two d_x buffers).
 * ------------------------------------------------------------------------- */
typedef struct ssm_backbone_dims {
  ssm_layer_dims layer; /* every layer's shape */
  int32_t n_layers;     /* >= 1 */
  int32_t input_dim;    /* width of the input embedding */
  int32_t keep;         /* SSM_KEEP_ALL or SSM_KEEP_INPUTS (activation memory plan) */
} ssm_backbone_dims;

/* What a training step keeps between the backbone's forward and backward:
 * SSM_KEEP_ALL: xs and every layer's saved activations (`saved`, with its
 *   optional h_ckpt), 455 MB per layer of the full layer shape;
 * SSM_KEEP_INPUTS: only xs (50 MB per layer); `saved` may be null, the forward
 *   writes each layer's activations into its workspace and drops them, and the
 *   backward runs each layer's forward again (into its workspace) just before
 *   that layer's backward: one more layer forward per layer for about 86 % less
 *   kept memory.  Results are the same bitwise (the same kernels rebuild the
 *   same activations). */
enum { SSM_KEEP_ALL = 0, SSM_KEEP_INPUTS = 1 };

size_t mamba_backbone_fwd_workspace_size(const ssm_backbone_dims* dims);
int mamba_backbone_fwd(const void* inp, const void* W_ip, const float* b_ip, const float* norm_f_w,
                       const ssm_layer_weights* layers, void* const* xs, const ssm_layer_saved* saved,
                       void* out, void* workspace, size_t ws_bytes, const ssm_backbone_dims* dims,
                       void* stream);
size_t mamba_backbone_bwd_workspace_size(const ssm_backbone_dims* dims);
int mamba_backbone_bwd(const void* inp, const void* W_ip, const float* norm_f_w,
                       const ssm_layer_weights* layers, const void* const* xs,
                       const ssm_layer_saved* saved, const void* d_out, void* d_inp,
                       const ssm_layer_grads* grads, float* d_W_ip, float* d_b_ip, float* d_norm_f_w,
                       int flags, void* workspace, size_t ws_bytes, const ssm_backbone_dims* dims,
                       void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SSMBWD_H */
