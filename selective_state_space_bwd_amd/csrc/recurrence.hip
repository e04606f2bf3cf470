// Reverse linear recurrence along t of time-major [B, T, C] tensors:
//
//   x_t = b_t + a_{t+1} x_{t+1},  x_T = 0      (inclusive; exclusive: x_t - b_t)
//
// the one-state adjoint sweep of mamba-rs 0.5.1 cpu/backward.rs Phase B3 (its
// d_h <- da * d_h), and with a = 1 the cumsum backward of rlx-cpu 0.2.17
// training_bwd.rs (cumsum_backward_row) along t.  It runs on the same segment
// machinery as the selective scan: a lane owns one (b, c) channel, time is cut
// into segments that run side by side, and the pair operator joins them:
//
//   1. summary (segments 1 .. n-1): walking the segment backwards from a zero
//      carry gives the carry it hands to the segment before it, V_s, and the
//      product of its decays, D_s (the carry entering from the right reaches
//      the segment's start scaled by D_s: c_{s-1} = V_s + D_s c_s);
//   2. carry (per channel): c over the segments, right to left;
//   3. final: each segment walks backwards again from its carry and writes x.
// No atomics; results are bitwise repeatable.
#include "common.hpp"

namespace ssm {

constexpr int kRsBlock = 256;  // channels per block
constexpr int kRsGroup = 8;    // steps whose loads are issued together

struct RsShape {
  int T, C, seg, nseg;
};

// one group of up to kRsGroup steps t = top, top - 1, .. (>= t0), values as float;
// steps below t0 repeat t0 (never used)
template <typename T>
__device__ __forceinline__ void rs_load(const T* __restrict__ p, size_t base, int C, int top, int t0,
                                        float (&v)[kRsGroup]) {
#pragma unroll
  for (int j = 0; j < kRsGroup; ++j) v[j] = ld(p, base + (size_t)max(top - j, t0) * C);
}

template <typename T, bool HAS_A>
__global__ __launch_bounds__(kRsBlock) void rs_summary(const T* __restrict__ a, const T* __restrict__ b,
                                                       float* __restrict__ V, float* __restrict__ Dp, RsShape sh) {
  const int c = blockIdx.x * kRsBlock + threadIdx.x;
  const int s = blockIdx.y + 1, bi = blockIdx.z;
  if (c >= sh.C) return;
  const int t0 = s * sh.seg, t1 = min(sh.T, t0 + sh.seg);
  const size_t base = (size_t)bi * sh.T * sh.C + c;
  float xc = 0.f, D = 1.f;
  for (int top = t1 - 1; top >= t0; top -= kRsGroup) {
    float bv[kRsGroup], av[kRsGroup];
    rs_load(b, base, sh.C, top, t0, bv);
    if (HAS_A) rs_load(a, base, sh.C, top, t0, av);
#pragma unroll
    for (int j = 0; j < kRsGroup; ++j) {
      if (top - j >= t0) {
        const float x = bv[j] + xc;
        xc = HAS_A ? av[j] * x : x;
        if (HAS_A) D *= av[j];
      }
    }
  }
  const size_t o = ((size_t)bi * sh.nseg + s) * sh.C + c;
  V[o] = xc;
  if (HAS_A) Dp[o] = D;
}

// in place: V[b, s] becomes the carry entering segment s from the right.  One
// thread per channel walks the segments; each group's loads are issued together
// (the carry chain itself is one fma per segment), and one-wave blocks spread the
// few channels over many CUs.
constexpr int kRsCarryBlock = 64;

template <bool HAS_A>
__global__ __launch_bounds__(kRsCarryBlock) void rs_carry(float* __restrict__ V, const float* __restrict__ Dp, int Bt,
                                                          RsShape sh) {
  const int idx = blockIdx.x * kRsCarryBlock + threadIdx.x;
  if (idx >= Bt * sh.C) return;
  const int bi = idx / sh.C, c = idx - bi * sh.C;
  const size_t o0 = (size_t)bi * sh.nseg * sh.C + c;
  float cin = 0.f;
  for (int top = sh.nseg - 1; top >= 1; top -= kRsGroup) {
    float v[kRsGroup], dp[kRsGroup];
#pragma unroll
    for (int j = 0; j < kRsGroup; ++j) {  // segments below 1 repeat segment 1 (never used)
      const size_t o = o0 + (size_t)max(top - j, 1) * sh.C;
      v[j] = V[o];
      dp[j] = HAS_A ? Dp[o] : 1.f;
    }
#pragma unroll
    for (int j = 0; j < kRsGroup; ++j) {
      if (top - j >= 1) {
        V[o0 + (size_t)(top - j) * sh.C] = cin;
        cin = HAS_A ? fmaf(dp[j], cin, v[j]) : v[j] + cin;
      }
    }
  }
  V[o0] = cin;
}

template <typename T, bool HAS_A, bool EXCL>
__global__ __launch_bounds__(kRsBlock) void rs_final(const T* __restrict__ a, const T* __restrict__ b,
                                                     T* __restrict__ x, const float* __restrict__ V, RsShape sh) {
  const int c = blockIdx.x * kRsBlock + threadIdx.x;
  const int s = blockIdx.y, bi = blockIdx.z;
  if (c >= sh.C) return;
  const int t0 = s * sh.seg, t1 = min(sh.T, t0 + sh.seg);
  const size_t base = (size_t)bi * sh.T * sh.C + c;
  float xc = sh.nseg > 1 ? V[((size_t)bi * sh.nseg + s) * sh.C + c] : 0.f;
  for (int top = t1 - 1; top >= t0; top -= kRsGroup) {
    float bv[kRsGroup], av[kRsGroup];
    rs_load(b, base, sh.C, top, t0, bv);
    if (HAS_A) rs_load(a, base, sh.C, top, t0, av);
#pragma unroll
    for (int j = 0; j < kRsGroup; ++j) {
      if (top - j >= t0) {
        const float full = bv[j] + xc;
        st(x, base + (size_t)(top - j) * sh.C, EXCL ? xc : full);
        xc = HAS_A ? av[j] * full : full;
      }
    }
  }
}

namespace {

// segments: enough blocks to give every CU several (at least 32 steps each)
RsShape rs_plan(int batch, int T, int C) {
  RsShape sh{};
  sh.T = T;
  sh.C = C;
  const long long tiles = (long long)((C + kRsBlock - 1) / kRsBlock) * batch;
  const long long want = (2048 + tiles - 1) / tiles;
  const long long most = (T + 31) / 32;
  const long long nseg = want < 1 ? 1 : (want > most ? (most < 1 ? 1 : most) : want);
  sh.seg = (int)((T + nseg - 1) / nseg);
  if (sh.seg < 1) sh.seg = 1;
  sh.nseg = (T + sh.seg - 1) / sh.seg;
  return sh;
}

size_t rs_workspace(int batch, const RsShape& sh, bool has_a) {
  if (sh.nseg <= 1) return 0;
  const size_t n = (size_t)batch * sh.nseg * sh.C;
  return align_up(n * sizeof(float)) * (has_a ? 2 : 1);
}

template <typename T>
void rs_launch(const void* a, const void* b, void* x, int batch, const RsShape& sh, bool excl, float* V, float* Dp,
               hipStream_t st) {
  const T* ta = static_cast<const T*>(a);
  const T* tb = static_cast<const T*>(b);
  T* tx = static_cast<T*>(x);
  const int ntile = (sh.C + kRsBlock - 1) / kRsBlock;
  if (sh.nseg > 1) {
    const dim3 g1(ntile, sh.nseg - 1, batch);
    const int nc = (int)(((long long)batch * sh.C + kRsCarryBlock - 1) / kRsCarryBlock);
    if (a) {
      hipLaunchKernelGGL((rs_summary<T, true>), g1, dim3(kRsBlock), 0, st, ta, tb, V, Dp, sh);
      hipLaunchKernelGGL((rs_carry<true>), dim3(nc), dim3(kRsCarryBlock), 0, st, V, Dp, batch, sh);
    } else {
      hipLaunchKernelGGL((rs_summary<T, false>), g1, dim3(kRsBlock), 0, st, ta, tb, V, Dp, sh);
      hipLaunchKernelGGL((rs_carry<false>), dim3(nc), dim3(kRsCarryBlock), 0, st, V, Dp, batch, sh);
    }
  }
  const dim3 g3(ntile, sh.nseg, batch);
#define RS_FINAL(HA, EX) hipLaunchKernelGGL((rs_final<T, HA, EX>), g3, dim3(kRsBlock), 0, st, ta, tb, tx, V, sh)
  if (a) {
    if (excl) RS_FINAL(true, true);
    else RS_FINAL(true, false);
  } else {
    if (excl) RS_FINAL(false, true);
    else RS_FINAL(false, false);
  }
#undef RS_FINAL
}

}  // namespace
}  // namespace ssm

using namespace ssm;

extern "C" size_t reverse_linear_scan_workspace_size(int batch, int seqlen, int channels, int has_a) {
  if (batch <= 0 || seqlen <= 0 || channels <= 0) return 0;
  return rs_workspace(batch, rs_plan(batch, seqlen, channels), has_a != 0);
}

extern "C" int reverse_linear_scan(const void* a, const void* b, void* x, int batch, int seqlen, int channels,
                                   int exclusive, void* workspace, size_t ws_bytes, int dtype, void* stream) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (batch < 0 || seqlen < 0 || channels < 0)
    return fail(SSM_ERR_INVALID_ARG, "bad size (batch %d seqlen %d channels %d)", batch, seqlen, channels);
  if ((size_t)batch * seqlen * channels == 0) return SSM_OK;
  if (!b || !x) return fail(SSM_ERR_INVALID_ARG, "b and x are required");
  if ((double)seqlen * channels * batch > 9.0e15) return fail(SSM_ERR_INVALID_ARG, "tensor too large");
  // batch is a grid dimension (<= 65535) and one carry thread runs per (batch, channel)
  if (batch > 65535 || (long long)batch * channels >= (1LL << 31))
    return fail(SSM_ERR_INVALID_ARG, "batch %d x channels %d beyond the supported range", batch, channels);
  const RsShape sh = rs_plan(batch, seqlen, channels);
  const size_t need = rs_workspace(batch, sh, a != nullptr);
  if (need && (!workspace || ws_bytes < need || !aligned256(workspace)))
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed (256-byte aligned)",
                workspace ? ws_bytes : 0, need);
  float* V = static_cast<float*>(workspace);
  // decay products in the second half of the workspace when a is given
  float* Dp = (need && a) ? reinterpret_cast<float*>(static_cast<char*>(workspace) + need / 2) : nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == SSM_F32) rs_launch<float>(a, b, x, batch, sh, exclusive != 0, V, Dp, st);
  else rs_launch<bf16>(a, b, x, batch, sh, exclusive != 0, V, Dp, st);
  return check_launch("reverse_linear_scan");
}
