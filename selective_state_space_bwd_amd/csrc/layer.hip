// The Mamba layer around the scan: forward (to build the saved activations) and
// the backward of mamba-rs cpu/backward.rs backward_mamba_layer_batched,
// Phases B1-B8, as a sequence of this library's kernels on one stream:
//
//   B1  out_proj     d_gated = d_out W_out,  dW_out = d_out^T gated   (gated recomputed from y, z)
//   B2+B3 gate and scan backward with the softplus epilogue:
//                    d_u, d_raw, d_A_log, d_D, d_z (into d_xz), d_B | d_C (into d_xdbl)
//   B4  dt_proj      d_dt_in (into d_xdbl), dW_dt, db_dt
//   B5  x_proj       d_u += d_xdbl W_x,  dW_x = d_xdbl^T u            (u recomputed from x_b)
//   B6  SiLU + conv  d_x_b (into d_xz), d_conv_w, d_conv_b
//   B7  in_proj      d_xn = d_xz W_in,  dW_in = d_xz^T xn             (xn recomputed from x)
//   B8  RMSNorm      d_x = RMSNorm'(d_xn) + d_out (residual), d_norm_w
//
// Every intermediate lives in the caller's workspace; nothing is allocated here.
#include <initializer_list>

#include "common.hpp"

using namespace ssm;

namespace {

struct Carver {
  char* base;
  size_t off = 0;
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  }
};

ssm_dims scan_dims_of(const ssm_layer_dims& d) {
  ssm_dims s{};
  s.batch = d.batch;
  s.seqlen = d.seqlen;
  s.d_inner = d.d_inner;
  s.d_state = d.d_state;
  s.ld_bc = d.dt_rank + 2 * d.d_state;
  s.ld_dbc = s.ld_bc;
  s.seg_len = d.seg_len;
  s.ld_z = 2 * d.d_inner;
  return s;
}

int check_layer(const ssm_layer_dims* d) {
  if (!d) return fail(SSM_ERR_INVALID_ARG, "dims is null");
  if (d->batch <= 0 || d->seqlen <= 0 || d->d_model <= 0 || d->d_inner <= 0 || d->dt_rank <= 0 || d->d_conv <= 0)
    return fail(SSM_ERR_INVALID_ARG, "layer sizes must be positive (batch %d seqlen %d d_model %d d_inner %d "
                "dt_rank %d d_conv %d)", d->batch, d->seqlen, d->d_model, d->d_inner, d->dt_rank, d->d_conv);
  if (d->d_state != 4 && d->d_state != 8 && d->d_state != 16)
    return fail(SSM_ERR_UNSUPPORTED, "d_state %d not in {4, 8, 16}", d->d_state);
  if ((d->d_model | d->d_inner | d->dt_rank) & 7)
    return fail(SSM_ERR_UNSUPPORTED, "d_model, d_inner and dt_rank must be multiples of 8");
  if (d->d_conv > 8) return fail(SSM_ERR_UNSUPPORTED, "d_conv %d > 8", d->d_conv);
  if (d->d_model > 4096) return fail(SSM_ERR_UNSUPPORTED, "d_model %d > 4096", d->d_model);
  if (!(d->eps >= 0.f)) return fail(SSM_ERR_INVALID_ARG, "eps must be >= 0");
  if ((double)d->batch * d->seqlen * 2.0 * d->d_inner >= 9.0e15 || (double)d->batch * d->seqlen >= 2147483648.0)
    return fail(SSM_ERR_INVALID_ARG, "layer too large");
  // the scan's own checks (segment length, row strides inside the layer's rows),
  // so that no stage has launched when one of them fails
  const ssm_dims sd = scan_dims_of(*d);
  return scan_check_dims(&sd, SSM_BF16);
}

int check_weights(const ssm_layer_weights* w) {
  if (!w || !w->norm_w || !w->W_in || !w->conv_w || !w->W_x || !w->W_dt || !w->A_log || !w->D || !w->W_out)
    return fail(SSM_ERR_INVALID_ARG, "a weight pointer is null (only conv_b and b_dt may be)");
  if (!aligned16(w->W_in) || !aligned16(w->W_x) || !aligned16(w->W_dt) || !aligned16(w->W_out))
    return fail(SSM_ERR_UNSUPPORTED, "weight matrices must be 16-byte aligned");
  return SSM_OK;
}

int check_saved(const ssm_layer_saved* s) {
  if (!s || !s->xz || !s->xdbl || !s->delta || (!s->y && !s->gated))
    return fail(SSM_ERR_INVALID_ARG, "a saved activation is null (y may be null only when gated is given)");
  const void* opt[] = {s->y, s->h_ckpt, s->gated, s->u, s->xn};
  bool ok = aligned16(s->xz) && aligned16(s->xdbl) && aligned16(s->delta);
  for (const void* p : opt) ok = ok && (!p || aligned16(p));
  if (!ok) return fail(SSM_ERR_UNSUPPORTED, "activations must be 16-byte aligned");
  return SSM_OK;
}


size_t max_of(std::initializer_list<size_t> v) {
  size_t m = 0;
  for (size_t x : v) m = x > m ? x : m;
  return m;
}

// scratch shared by the stages (they run one after another on the stream)
size_t fwd_scratch(const ssm_layer_dims& d) {
  const int64_t M = (int64_t)d.batch * d.seqlen;
  const int R2 = d.dt_rank + 2 * d.d_state;
  const ssm_dims sd = scan_dims_of(d);
  return max_of({linear_fwd_workspace_size(M, d.d_model, 2 * d.d_inner), linear_fwd_workspace_size(M, d.d_inner, R2),
                 linear_fwd_workspace_size(M, d.dt_rank, d.d_inner), linear_fwd_workspace_size(M, d.d_inner, d.d_model),
                 ssm_scan_fwd_workspace_size(&sd, SSM_BF16)});
}

size_t bwd_scratch(const ssm_layer_dims& d) {
  const int64_t M = (int64_t)d.batch * d.seqlen;
  const int R2 = d.dt_rank + 2 * d.d_state;
  const ssm_dims sd = scan_dims_of(d);
  return max_of({linear_bwd_workspace_size(M, d.d_inner, d.d_model), linear_bwd_workspace_size(M, d.dt_rank, d.d_inner),
                 linear_bwd_workspace_size(M, d.d_inner, R2), linear_bwd_workspace_size(M, d.d_model, 2 * d.d_inner),
                 ssm_scan_bwd_workspace_size(&sd, SSM_BF16),
                 conv1d_bwd_workspace_size(d.batch, d.seqlen, d.d_inner, d.d_conv),
                 rmsnorm_bwd_workspace_size(M, d.d_model)});
}

struct FwdBufs {
  bf16 *xn, *u, *gated;
  void* scratch;
  size_t scratch_bytes;
};

FwdBufs carve_fwd(const ssm_layer_dims& d, void* ws, size_t* total) {
  const size_t M = (size_t)d.batch * d.seqlen;
  Carver c{static_cast<char*>(ws)};
  FwdBufs b{};
  b.xn = static_cast<bf16*>(c.take(M * d.d_model * 2));
  b.u = static_cast<bf16*>(c.take(M * d.d_inner * 2));
  b.gated = static_cast<bf16*>(c.take(M * d.d_inner * 2));
  b.scratch_bytes = fwd_scratch(d);
  b.scratch = c.take(b.scratch_bytes);
  *total = c.off;
  return b;
}

struct BwdBufs {
  bf16 *gated, *d_gated, *u, *d_u, *d_raw, *d_xdbl, *d_xz, *xn, *d_xn;
  void* scratch;
  size_t scratch_bytes;
};

BwdBufs carve_bwd(const ssm_layer_dims& d, void* ws, size_t* total) {
  const size_t M = (size_t)d.batch * d.seqlen;
  const size_t di = d.d_inner, R2 = d.dt_rank + 2 * d.d_state;
  Carver c{static_cast<char*>(ws)};
  BwdBufs b{};
  b.gated = static_cast<bf16*>(c.take(M * di * 2));
  b.d_raw = b.gated;  // gated is dead once dW_out is formed, before the scan writes d_raw
  b.d_gated = static_cast<bf16*>(c.take(M * di * 2));
  b.u = static_cast<bf16*>(c.take(M * di * 2));
  b.d_u = static_cast<bf16*>(c.take(M * di * 2));
  b.d_xdbl = static_cast<bf16*>(c.take(M * R2 * 2));
  b.d_xz = static_cast<bf16*>(c.take(M * 2 * di * 2));
  b.xn = static_cast<bf16*>(c.take(M * d.d_model * 2));
  b.d_xn = static_cast<bf16*>(c.take(M * d.d_model * 2));
  b.scratch_bytes = bwd_scratch(d);
  b.scratch = c.take(b.scratch_bytes);
  *total = c.off;
  return b;
}

void mark(void* const* ev, int k, hipStream_t st) {
  if (ev && ev[k]) (void)hipEventRecord(static_cast<hipEvent_t>(ev[k]), st);
}

#define TRY(expr)                 \
  do {                            \
    const int rc_ = (expr);       \
    if (rc_ != SSM_OK) return rc_; \
  } while (0)

}  // namespace

extern "C" size_t mamba_layer_fwd_workspace_size(const ssm_layer_dims* dims) {
  if (!dims || check_layer(dims) != SSM_OK) return 0;
  size_t total = 0;
  carve_fwd(*dims, nullptr, &total);
  return total;
}

extern "C" int mamba_layer_fwd(const void* x, const ssm_layer_weights* w, void* out, const ssm_layer_saved* saved,
                               void* workspace, size_t ws_bytes, const ssm_layer_dims* dims, void* stream) {
  TRY(check_layer(dims));
  TRY(check_weights(w));
  TRY(check_saved(saved));
  if (!x || !out || !aligned16(x) || !aligned16(out)) return fail(SSM_ERR_INVALID_ARG, "x / out null or misaligned");
  const ssm_layer_dims& d = *dims;
  size_t need = 0;
  const FwdBufs b = carve_fwd(d, workspace, &need);
  if (!workspace || ws_bytes < need || !aligned256(workspace))
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed (256-byte aligned)",
                workspace ? ws_bytes : 0, need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t M = (int64_t)d.batch * d.seqlen;
  const int dm = d.d_model, di = d.d_inner, R = d.dt_rank, N = d.d_state, R2 = R + 2 * N;
  bf16* xz = static_cast<bf16*>(saved->xz);
  bf16* xdbl = static_cast<bf16*>(saved->xdbl);
  bf16* delta = static_cast<bf16*>(saved->delta);
  // the products' inputs go to the caller's buffers when it keeps them, else to the workspace
  bf16* xn = saved->xn ? static_cast<bf16*>(saved->xn) : b.xn;
  bf16* u = saved->u ? static_cast<bf16*>(saved->u) : b.u;
  bf16* gated = saved->gated ? static_cast<bf16*>(saved->gated) : b.gated;
  // every product's arguments are checked before the first launch
  TRY(gemm_check(xn, dm, w->W_in, dm, xz, (int)M, 2 * di, dm, b.scratch_bytes, b.scratch));
  TRY(gemm_check(u, di, w->W_x, di, xdbl, (int)M, R2, di, b.scratch_bytes, b.scratch));
  TRY(gemm_check(xdbl, R2, w->W_dt, R, delta, (int)M, di, R, b.scratch_bytes, b.scratch));
  TRY(gemm_check(gated, di, w->W_out, di, out, (int)M, dm, di, b.scratch_bytes, b.scratch));

  launch_rmsnorm_fwd(static_cast<const bf16*>(x), w->norm_w, xn, M, dm, d.eps, st);
  gemm_bf16(xn, true, dm, w->W_in, true, dm, xz, 2 * di, SSM_BF16, (int)M, 2 * di, dm, 0, b.scratch, st);
  launch_conv_silu_fwd(xz, 2 * di, w->conv_w, w->conv_b, u, di, d.batch, d.seqlen, di, d.d_conv, st);
  gemm_bf16(u, true, di, w->W_x, true, di, xdbl, R2, SSM_BF16, (int)M, R2, di, 0, b.scratch, st);
  gemm_bf16(xdbl, true, R2, w->W_dt, true, R, delta, di, SSM_BF16, (int)M, di, R, 0, b.scratch, st);
  launch_bias_softplus(delta, w->b_dt, M, di, st);
  const ssm_dims sd = scan_dims_of(d);
  TRY(ssm_scan_fwd(u, delta, w->A_log, xdbl + R, xdbl + R + N, w->D, xz + di, saved->y, gated, saved->h_ckpt,
                   saved->h_ckpt ? 8 : 0, b.scratch, b.scratch_bytes, &sd, SSM_BF16, stream));
  // residual: out = x, then out += gated W_out^T
  if (hipMemcpyAsync(out, x, (size_t)M * dm * 2, hipMemcpyDeviceToDevice, st) != hipSuccess)
    return fail(SSM_ERR_LAUNCH, "residual copy failed");
  gemm_bf16(gated, true, di, w->W_out, true, di, out, dm, SSM_BF16, (int)M, dm, di, 1, b.scratch, st);
  return check_launch("mamba_layer_fwd");
}

extern "C" size_t mamba_layer_bwd_workspace_size(const ssm_layer_dims* dims) {
  if (!dims || check_layer(dims) != SSM_OK) return 0;
  size_t total = 0;
  carve_bwd(*dims, nullptr, &total);
  return total;
}

extern "C" int mamba_layer_bwd_timed(const void* x, const ssm_layer_weights* w, const ssm_layer_saved* saved,
                                     const void* d_out, void* d_x, const ssm_layer_grads* g, void* workspace,
                                     size_t ws_bytes, const ssm_layer_dims* dims, void* stream,
                                     void* const* ev) {
  TRY(check_layer(dims));
  TRY(check_weights(w));
  TRY(check_saved(saved));
  if (!x || !d_out || !d_x || !aligned16(x) || !aligned16(d_out))
    return fail(SSM_ERR_INVALID_ARG, "x, d_out or d_x null or misaligned");
  if (!g || !g->d_norm_w || !g->d_W_in || !g->d_conv_w || !g->d_conv_b || !g->d_W_x || !g->d_W_dt || !g->d_b_dt ||
      !g->d_A_log || !g->d_D || !g->d_W_out)
    return fail(SSM_ERR_INVALID_ARG, "a gradient pointer is null");
  const ssm_layer_dims& d = *dims;
  size_t need = 0;
  const BwdBufs b = carve_bwd(d, workspace, &need);
  if (!workspace || ws_bytes < need || !aligned256(workspace))
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed (256-byte aligned)",
                workspace ? ws_bytes : 0, need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t M = (int64_t)d.batch * d.seqlen;
  const int dm = d.d_model, di = d.d_inner, R = d.dt_rank, N = d.d_state, R2 = R + 2 * N;
  const bf16* xz = static_cast<const bf16*>(saved->xz);
  const bf16* xdbl = static_cast<const bf16*>(saved->xdbl);
  const ssm_dims sd = scan_dims_of(d);
  void* sc = b.scratch;
  const size_t scb = b.scratch_bytes;
  // the products' inputs: kept by the forward, or recomputed into the workspace below
  const bf16* gated = saved->gated ? static_cast<const bf16*>(saved->gated) : b.gated;
  const bf16* u = saved->u ? static_cast<const bf16*>(saved->u) : b.u;
  const bf16* xn = saved->xn ? static_cast<const bf16*>(saved->xn) : b.xn;

  mark(ev, 0, st);
  if (!saved->gated) launch_gate_fwd(static_cast<const bf16*>(saved->y), xz + di, 2 * di, b.gated, M, di, st);
  mark(ev, 1, st);
  // B1: out = gated W_out^T (+ x)
  const int acc = g->accumulate ? SSM_BWD_ACCUMULATE : 0;
  TRY(linear_bwd(gated, di, w->W_out, d_out, dm, b.d_gated, di, acc, g->d_W_out, nullptr, M, di, dm, sc, scb,
                 SSM_BF16, stream));
  mark(ev, 2, st);
  if (!saved->u) launch_conv_silu_fwd(xz, 2 * di, w->conv_w, w->conv_b, b.u, di, d.batch, d.seqlen, di, d.d_conv, st);
  mark(ev, 3, st);
  // B2 + B3 (+ softplus backward): d_z lands in the second half of d_xz, d_B | d_C in d_xdbl
  if (saved->h_ckpt)
    TRY(ssm_scan_bwd_ckpt(u, saved->delta, w->A_log, xdbl + R, xdbl + R + N, w->D, xz + di, b.d_gated,
                          saved->h_ckpt, b.d_u, b.d_raw, g->d_A_log, b.d_xdbl + R, b.d_xdbl + R + N, g->d_D,
                          b.d_xz + di, SSM_BWD_SOFTPLUS | acc, sc, scb, &sd, SSM_BF16, stream, nullptr));
  else
    TRY(ssm_scan_bwd(u, saved->delta, w->A_log, xdbl + R, xdbl + R + N, w->D, xz + di, b.d_gated, b.d_u, b.d_raw,
                     g->d_A_log, b.d_xdbl + R, b.d_xdbl + R + N, g->d_D, b.d_xz + di, SSM_BWD_SOFTPLUS | acc, sc, scb,
                     &sd, SSM_BF16, stream));
  mark(ev, 4, st);
  // B4: raw = dt_in W_dt^T + b_dt, dt_in = xdbl[:, :R]; d_dt_in fills d_xdbl[:, :R]
  TRY(linear_bwd(xdbl, R2, w->W_dt, b.d_raw, di, b.d_xdbl, R2, acc, g->d_W_dt, g->d_b_dt, M, R, di, sc, scb,
                 SSM_BF16, stream));
  mark(ev, 5, st);
  // B5: xdbl = u W_x^T; d_u collects the scan's and this product's parts
  TRY(linear_bwd(u, di, w->W_x, b.d_xdbl, R2, b.d_u, di, SSM_BWD_ACCUMULATE_DX | acc, g->d_W_x, nullptr, M, di,
                 R2, sc, scb, SSM_BF16,
                 stream));
  mark(ev, 6, st);
  // B6: SiLU + conv backward; d_x_b fills the first half of d_xz
  TRY(conv1d_bwd(xz, w->conv_w, w->conv_b, b.d_u, b.d_xz, g->d_conv_w, g->d_conv_b, d.batch, d.seqlen, di,
                 d.d_conv, 2 * di, di, 2 * di, acc, sc, scb, SSM_BF16, stream));
  mark(ev, 7, st);
  if (!saved->xn) launch_rmsnorm_fwd(static_cast<const bf16*>(x), w->norm_w, b.xn, M, dm, d.eps, st);
  mark(ev, 8, st);
  // B7: xz = xn W_in^T
  TRY(linear_bwd(xn, dm, w->W_in, b.d_xz, 2 * di, b.d_xn, dm, acc, g->d_W_in, nullptr, M, dm, 2 * di, sc, scb,
                 SSM_BF16, stream));
  mark(ev, 9, st);
  // B8: RMSNorm backward plus the residual path
  TRY(rmsnorm_bwd(x, w->norm_w, b.d_xn, d_out, d_x, g->d_norm_w, M, dm, d.eps, acc, sc, scb, SSM_BF16, stream));
  mark(ev, 10, st);
  return check_launch("mamba_layer_bwd");
}

extern "C" int mamba_layer_bwd(const void* x, const ssm_layer_weights* w, const ssm_layer_saved* saved,
                               const void* d_out, void* d_x, const ssm_layer_grads* g, void* workspace,
                               size_t ws_bytes, const ssm_layer_dims* dims, void* stream) {
  return mamba_layer_bwd_timed(x, w, saved, d_out, d_x, g, workspace, ws_bytes, dims, stream, nullptr);
}

// ---------------------------------------------------------------------------
// The backbone around the layers (mamba-rs cpu/backward.rs,
// backward_mamba_backbone_batched): forward x_0 = inp W_ip^T + b_ip, each layer
// x_{l+1} = layer_l(x_l), out = RMSNorm(x_L; norm_f_w); backward norm_f first,
// the layers in reverse, then the input projection.  Every argument is checked
// before the first launch.
namespace {

int check_backbone(const ssm_backbone_dims* bd) {
  if (!bd) return fail(SSM_ERR_INVALID_ARG, "dims is null");
  TRY(check_layer(&bd->layer));
  if (bd->n_layers < 1) return fail(SSM_ERR_INVALID_ARG, "n_layers %d < 1", bd->n_layers);
  if (bd->keep != SSM_KEEP_ALL && bd->keep != SSM_KEEP_INPUTS)
    return fail(SSM_ERR_INVALID_ARG, "keep %d is neither SSM_KEEP_ALL nor SSM_KEEP_INPUTS", bd->keep);
  if (bd->input_dim <= 0 || (bd->input_dim & 7))
    return fail(SSM_ERR_UNSUPPORTED, "input_dim %d must be a positive multiple of 8", bd->input_dim);
  return SSM_OK;
}

int check_layer_arrays(const ssm_backbone_dims* bd, const ssm_layer_weights* layers, const void* const* xs,
                       const ssm_layer_saved* saved) {
  const bool kept = bd->keep == SSM_KEEP_ALL;
  if (!layers || !xs || (kept && !saved)) return fail(SSM_ERR_INVALID_ARG, "layers, xs and saved are required");
  for (int l = 0; l < bd->n_layers; ++l) {
    TRY(check_weights(&layers[l]));
    if (kept) TRY(check_saved(&saved[l]));
  }
  for (int l = 0; l <= bd->n_layers; ++l)
    if (!xs[l] || !aligned16(xs[l])) return fail(SSM_ERR_INVALID_ARG, "xs[%d] null or misaligned", l);
  return SSM_OK;
}

size_t backbone_fwd_scratch(const ssm_backbone_dims& bd) {
  const int64_t M = (int64_t)bd.layer.batch * bd.layer.seqlen;
  return max_of({mamba_layer_fwd_workspace_size(&bd.layer), linear_fwd_workspace_size(M, bd.input_dim, bd.layer.d_model)});
}

size_t backbone_bwd_scratch(const ssm_backbone_dims& bd) {
  const int64_t M = (int64_t)bd.layer.batch * bd.layer.seqlen;
  size_t s = max_of({mamba_layer_bwd_workspace_size(&bd.layer), rmsnorm_bwd_workspace_size(M, bd.layer.d_model),
                     linear_bwd_workspace_size(M, bd.input_dim, bd.layer.d_model)});
  if (bd.keep == SSM_KEEP_INPUTS) s = max_of({s, mamba_layer_fwd_workspace_size(&bd.layer)});
  return s;
}

// With SSM_KEEP_INPUTS, one layer's saved activations and its (recomputed)
// output live in the workspace, reused by every layer in turn.
struct LayerKeep {
  ssm_layer_saved saved;
  void* out;
};

LayerKeep carve_keep(const ssm_layer_dims& d, void* ws, size_t* total) {
  const size_t M = (size_t)d.batch * d.seqlen;
  Carver c{static_cast<char*>(ws)};
  LayerKeep k{};
  k.saved.xz = c.take(M * 2 * d.d_inner * 2);
  k.saved.xdbl = c.take(M * (d.dt_rank + 2 * d.d_state) * 2);
  k.saved.delta = c.take(M * d.d_inner * 2);
  k.saved.y = c.take(M * d.d_inner * 2);
  k.saved.h_ckpt = nullptr;
  k.out = c.take(M * d.d_model * 2);
  *total = c.off;
  return k;
}

size_t keep_bytes(const ssm_backbone_dims& bd) {
  if (bd.keep != SSM_KEEP_INPUTS) return 0;
  size_t total = 0;
  carve_keep(bd.layer, nullptr, &total);
  return total;
}

}  // namespace

extern "C" size_t mamba_backbone_fwd_workspace_size(const ssm_backbone_dims* dims) {
  if (!dims || check_backbone(dims) != SSM_OK) return 0;
  return keep_bytes(*dims) + backbone_fwd_scratch(*dims);
}

extern "C" int mamba_backbone_fwd(const void* inp, const void* W_ip, const float* b_ip, const float* norm_f_w,
                                  const ssm_layer_weights* layers, void* const* xs, const ssm_layer_saved* saved,
                                  void* out, void* workspace, size_t ws_bytes, const ssm_backbone_dims* dims,
                                  void* stream) {
  TRY(check_backbone(dims));
  const ssm_backbone_dims& bd = *dims;
  TRY(check_layer_arrays(dims, layers, xs, saved));
  if (!inp || !W_ip || !norm_f_w || !out || !aligned16(out)) return fail(SSM_ERR_INVALID_ARG, "a pointer is null");
  const int64_t M = (int64_t)bd.layer.batch * bd.layer.seqlen;
  const int dm = bd.layer.d_model, L = bd.n_layers;
  const size_t kb = keep_bytes(bd);
  const size_t need = kb + backbone_fwd_scratch(bd);
  if (!workspace || ws_bytes < need || !aligned256(workspace))
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed (256-byte aligned)",
                workspace ? ws_bytes : 0, need);
  size_t unused = 0;
  const LayerKeep keep = carve_keep(bd.layer, workspace, &unused);   // used with SSM_KEEP_INPUTS only
  void* sc = static_cast<char*>(workspace) + kb;
  const size_t scb = ws_bytes - kb;
  TRY(gemm_check(inp, bd.input_dim, W_ip, bd.input_dim, xs[0], (int)M, dm, bd.input_dim, scb, sc));
  hipStream_t st = static_cast<hipStream_t>(stream);
  TRY(linear_fwd(inp, bd.input_dim, W_ip, nullptr, xs[0], dm, M, bd.input_dim, dm, sc, scb, SSM_BF16, stream));
  if (b_ip) launch_bias_add(static_cast<bf16*>(xs[0]), b_ip, M, dm, st);
  for (int l = 0; l < L; ++l)
    TRY(mamba_layer_fwd(xs[l], &layers[l], xs[l + 1], kb ? &keep.saved : &saved[l], sc, scb, &bd.layer, stream));
  launch_rmsnorm_fwd(static_cast<const bf16*>(xs[L]), norm_f_w, static_cast<bf16*>(out), M, dm, bd.layer.eps, st);
  return check_launch("mamba_backbone_fwd");
}

extern "C" size_t mamba_backbone_bwd_workspace_size(const ssm_backbone_dims* dims) {
  if (!dims || check_backbone(dims) != SSM_OK) return 0;
  const size_t grad = align_up((size_t)dims->layer.batch * dims->layer.seqlen * dims->layer.d_model * 2);
  return 2 * grad + keep_bytes(*dims) + backbone_bwd_scratch(*dims);
}

extern "C" int mamba_backbone_bwd(const void* inp, const void* W_ip, const float* norm_f_w,
                                  const ssm_layer_weights* layers, const void* const* xs,
                                  const ssm_layer_saved* saved, const void* d_out, void* d_inp,
                                  const ssm_layer_grads* grads, float* d_W_ip, float* d_b_ip, float* d_norm_f_w,
                                  int flags, void* workspace, size_t ws_bytes, const ssm_backbone_dims* dims,
                                  void* stream) {
  TRY(check_backbone(dims));
  const ssm_backbone_dims& bd = *dims;
  TRY(check_layer_arrays(dims, layers, xs, saved));
  if (flags & ~SSM_BWD_ACCUMULATE) return fail(SSM_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (!inp || !W_ip || !norm_f_w || !d_out || !aligned16(d_out) || !grads || !d_W_ip || !d_b_ip || !d_norm_f_w)
    return fail(SSM_ERR_INVALID_ARG, "a pointer is null");
  for (int l = 0; l < bd.n_layers; ++l) {
    const ssm_layer_grads* g = &grads[l];
    if (!g->d_norm_w || !g->d_W_in || !g->d_conv_w || !g->d_conv_b || !g->d_W_x || !g->d_W_dt || !g->d_b_dt ||
        !g->d_A_log || !g->d_D || !g->d_W_out)
      return fail(SSM_ERR_INVALID_ARG, "a gradient pointer of layer %d is null", l);
  }
  const int64_t M = (int64_t)bd.layer.batch * bd.layer.seqlen;
  const int dm = bd.layer.d_model, L = bd.n_layers;
  const size_t grad = align_up((size_t)M * dm * 2);
  const size_t kb = keep_bytes(bd);
  const size_t need = 2 * grad + kb + backbone_bwd_scratch(bd);
  if (!workspace || ws_bytes < need || !aligned256(workspace))
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed (256-byte aligned)",
                workspace ? ws_bytes : 0, need);
  char* base = static_cast<char*>(workspace);
  void* dbuf[2] = {base, base + grad};
  size_t unused = 0;
  const LayerKeep keep = carve_keep(bd.layer, base + 2 * grad, &unused);   // used with SSM_KEEP_INPUTS only
  void* sc = base + 2 * grad + kb;
  const size_t scb = ws_bytes - 2 * grad - kb;
  // the input projection's products (run last) are checked here, before anything is launched
  TRY(gemm_check(d_out, dm, W_ip, bd.input_dim, d_inp ? d_inp : d_out, (int)M, bd.input_dim, dm, scb, sc));
  TRY(gemm_check(d_out, dm, inp, bd.input_dim, d_W_ip, dm, bd.input_dim, (int)M, scb, sc));
  const int acc = flags & SSM_BWD_ACCUMULATE;
  // norm_f: d x_L (no residual here; each layer's backward adds its own)
  TRY(rmsnorm_bwd(xs[L], norm_f_w, d_out, nullptr, dbuf[0], d_norm_f_w, M, dm, bd.layer.eps, acc, sc, scb, SSM_BF16,
                  stream));
  int cur = 0;
  for (int l = L - 1; l >= 0; --l) {
    ssm_layer_grads g = grads[l];
    if (acc) g.accumulate = 1;
    // SSM_KEEP_INPUTS: this layer's activations again, from its kept input
    if (kb) TRY(mamba_layer_fwd(xs[l], &layers[l], keep.out, &keep.saved, sc, scb, &bd.layer, stream));
    const ssm_layer_saved* sv = kb ? &keep.saved : &saved[l];
    TRY(mamba_layer_bwd(xs[l], &layers[l], sv, dbuf[cur], dbuf[cur ^ 1], &g, sc, scb, &bd.layer, stream));
    cur ^= 1;
  }
  // input projection: dW_ip, db_ip (and d_inp if asked)
  TRY(linear_bwd(inp, bd.input_dim, W_ip, dbuf[cur], dm, d_inp, bd.input_dim, acc, d_W_ip, d_b_ip, M, bd.input_dim,
                 dm, sc, scb, SSM_BF16, stream));
  return check_launch("mamba_backbone_bwd");
}
