// The layer's bandwidth-bound backward pieces around the scan:
//   gating_bwd  — mamba-rs cpu/backward.rs Phase B2 on its own;
//   conv1d_bwd  — Phase B6: SiLU backward on the conv output fused with the
//                 causal depthwise conv backward;
//   rmsnorm_bwd — rlx-cpu training_bwd.rs rms_norm_backward_row (no shift term)
//                 with Phase B8's residual add.
// and the forward pieces a layer backward recomputes instead of storing
// (RMSNorm output, conv + SiLU output, the gated scan output) plus the dt_proj
// bias + softplus that turns the dt_proj product into delta.
// Reductions over rows / steps go to fixed-order partials, no atomics.
#include "common.hpp"

namespace ssm {

constexpr int kPwBlock = 256;

// 16 bytes of a row (8 bf16 or 4 float channels) held as float
template <typename T>
struct Vec16 {
  static constexpr int N = 16 / sizeof(T);
  float v[N];
  __device__ __forceinline__ void load(const T* __restrict__ p) { set(*reinterpret_cast<const uint4*>(p)); }
  __device__ __forceinline__ void set(const uint4 w) {
    if constexpr (sizeof(T) == 4) {
      v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y); v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
    } else {
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(u[i] << 16);
        v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
      }
    }
  }
  __device__ __forceinline__ void store(T* __restrict__ p) const {
    uint4 w;
    if constexpr (sizeof(T) == 4) {
      w = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
    } else {
      uint32_t u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        u[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
      w = make_uint4(u[0], u[1], u[2], u[3]);
    }
    *reinterpret_cast<uint4*>(p) = w;
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(kPwBlock) void fill_zero_f32(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kPwBlock + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kPwBlock) void gating_bwd_kernel(const T* __restrict__ dout, const T* __restrict__ y,
                                                              const T* __restrict__ z, T* __restrict__ dy,
                                                              T* __restrict__ dz, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kPwBlock;
  for (int64_t i = (int64_t)blockIdx.x * kPwBlock + threadIdx.x; i < n; i += stride) {
    const float g = ld(dout, i), yy = ld(y, i), zz = ld(z, i);
    const float s = sigmoid(zz);
    st(dy, i, g * zz * s);
    st(dz, i, g * yy * s * (1.f + zz * (1.f - s)));
  }
}

// ---------------------------------------------------------------------------
// conv1d: one thread per (b, chunk of kConvT steps, channel); the conv output
// and its SiLU derivative are rebuilt from x on the fly over a window of K taps.
constexpr int kConvT = 64;
constexpr int kMaxTaps = 8;

template <typename T, int K>
__global__ __launch_bounds__(kPwBlock) void conv1d_bwd_kernel(
    const T* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    const T* __restrict__ d_u, T* __restrict__ d_x, float* __restrict__ part, int Bt, int Tn, int Di,
    int ld_x, int ld_du, int ld_dx, int nchunk) {
  const int d = blockIdx.x * kPwBlock + threadIdx.x;
  const int c = blockIdx.y, b = blockIdx.z;
  if (d >= Di) return;
  float wk[K];
#pragma unroll
  for (int k = 0; k < K; ++k) wk[k] = w[(size_t)d * K + k];
  const float bd = bias ? bias[d] : 0.f;
  const int t0 = c * kConvT, t1 = min(Tn, t0 + kConvT);
  const size_t rx = (size_t)b * Tn;
  // window xs[k] = x[t - (K-1) + k] for the current t; gs[k] = g[t - (K-1) + k]
  float xs[K], gs[K], dw[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int tt = t0 - K + k;  // the window of step t0 - 1; x[t0] is shifted in by the loop
    xs[k] = tt >= 0 ? ld(x, (rx + tt) * ld_x + d) : 0.f;
    gs[k] = 0.f;
    dw[k] = 0.f;
  }
  float db = 0.f;
  const int tend = min(Tn, t1 + K - 1);
  for (int t = t0; t < tend; ++t) {
    // shift in x[t]
#pragma unroll
    for (int k = 0; k < K - 1; ++k) xs[k] = xs[k + 1];
    xs[K - 1] = ld(x, (rx + t) * ld_x + d);
    float cv = bd;
#pragma unroll
    for (int k = 0; k < K; ++k) cv = fmaf(wk[k], xs[k], cv);
    const float s = sigmoid(cv);
    const float g = ld(d_u, (rx + t) * ld_du + d) * s * (1.f + cv * (1.f - s));
#pragma unroll
    for (int k = 0; k < K - 1; ++k) gs[k] = gs[k + 1];
    gs[K - 1] = g;
    if (t < t1) {  // this chunk owns g[t] for the weight and bias sums
#pragma unroll
      for (int k = 0; k < K; ++k) dw[k] = fmaf(g, xs[k], dw[k]);
      db += g;
    }
    const int to = t - (K - 1);  // d_x[to] = sum_k g[to + K-1-k] w[k] = sum_k gs[K-1-k] w[k]
    if (to >= t0) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < K; ++k) acc = fmaf(gs[K - 1 - k], wk[k], acc);
      st(d_x, (rx + to) * ld_dx + d, acc);
    }
  }
  // the last K-1 outputs of the chunk whose g window runs past the sequence end
  for (int to = max(t0, tend - (K - 1)); to < t1; ++to) {
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int tg = to + (K - 1) - k;
      const float gv = (tg < tend) ? gs[K - 1 - (tend - 1 - tg)] : 0.f;
      acc = fmaf(gv, wk[k], acc);
    }
    st(d_x, (rx + to) * ld_dx + d, acc);
  }
  const size_t p = ((size_t)b * nchunk + c) * (K + 1);
#pragma unroll
  for (int k = 0; k < K; ++k) part[(p + k) * Di + d] = dw[k];
  part[(p + K) * Di + d] = db;
}

// Vector form for rows of 16-byte vectors (d_inner, the strides and the bases
// multiples of 16 bytes): a block's four waves take one vector of channels per
// lane and four consecutive chunks of tv steps, one chunk per wave.  Each
// wave issues the loads of kConvLoad steps together, then runs them; the waves'
// weight and bias sums combine in LDS in a fixed order into one partial per
// block.  The K-1 steps after a chunk, needed for its last d_x outputs, are
// recomputed by the wave (with zero gradient past the sequence end).
constexpr int kConvWaves = kPwBlock / kWave;
constexpr int kConvLoad = 4;
constexpr int kConvMinTV = 16;  // the workspace is sized for 4 x 16 steps per block (kConvT)
static_assert(kConvWaves * kConvMinTV >= 64, "conv partials per sequence");
// Blocks a CU holds at once, from the kernels' register use (the backward's
// window, weight sums and load buffers take two waves per SIMD, the forward's
// four).
constexpr int kConvBwdBlocksPerCU = 2;
constexpr int kConvFwdBlocksPerCU = 4;

// Steps per wave of the vector conv kernels: the grid is (channel vectors /
// 64) x (seqlen / 4 tv) x batch blocks, and each wave also recomputes the K - 1
// steps after its chunk.  Picks tv, a multiple of the load group, that
// minimises (rounds of resident blocks) x (tv + K - 1); ties go to the longer
// chunk (fewer weight-sum partials).
int conv_steps_per_wave(int seqlen, int nx, int batch, int K, int blocks_per_cu) {
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  const long slots = (long)cus * blocks_per_cu;
  int best = kConvMinTV;
  long best_cost = -1;
  for (int tv = kConvMinTV; tv <= 256; tv += kConvLoad) {
    const long blocks = (long)nx * ((seqlen + kConvWaves * tv - 1) / (kConvWaves * tv)) * batch;
    const long cost = (blocks + slots - 1) / slots * (tv + K - 1);
    if (best_cost < 0 || cost <= best_cost) {
      best_cost = cost;
      best = tv;
    }
    if (kConvWaves * tv >= seqlen) break;
  }
  return best;
}

template <typename T, int K>
struct ConvWindow {
  static constexpr int V = Vec16<T>::N;
  float wk[K][V], bd[V], xs[K][V], gs[K][V];

  __device__ __forceinline__ void init(const float* __restrict__ w, const float* __restrict__ bias, int d0) {
#pragma unroll
    for (int i = 0; i < V; ++i) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        wk[k][i] = w[(size_t)(d0 + i) * K + k];
        gs[k][i] = 0.f;
      }
      bd[i] = bias ? bias[d0 + i] : 0.f;
    }
  }
  // shift x[t] in; returns the conv output per channel
  __device__ __forceinline__ void push_x(const Vec16<T>& xv, float (&cv)[V]) {
#pragma unroll
    for (int i = 0; i < V; ++i) {
#pragma unroll
      for (int k = 0; k + 1 < K; ++k) xs[k][i] = xs[k + 1][i];
      xs[K - 1][i] = xv.v[i];
      float c = bd[i];
#pragma unroll
      for (int k = 0; k < K; ++k) c = fmaf(wk[k][i], xs[k][i], c);
      cv[i] = c;
    }
  }
};

template <typename T, int K>
__global__ __launch_bounds__(kPwBlock) void conv1d_bwd_vec(
    const T* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    const T* __restrict__ d_u, T* __restrict__ d_x, float* __restrict__ part, int Tn, int Di,
    int ld_x, int ld_du, int ld_dx, int tv) {
  constexpr int V = Vec16<T>::N;
  __shared__ float red[kConvWaves - 1][(K + 1) * V][kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int d0 = (blockIdx.x * kWave + lane) * V;
  const bool on = d0 < Di;
  const int t0 = (blockIdx.y * kConvWaves + wave) * tv;
  const int t1 = min(Tn, t0 + tv);
  const size_t rx = (size_t)blockIdx.z * Tn;
  float dw[K + 1][V];  // K weight sums, then the bias sum
#pragma unroll
  for (int k = 0; k <= K; ++k)
#pragma unroll
    for (int i = 0; i < V; ++i) dw[k][i] = 0.f;

  if (on && t0 < Tn) {
    ConvWindow<T, K> win;
    win.init(w, bias, d0);
#pragma unroll
    for (int k = 1; k < K; ++k) {  // x[t0 - K + k]; slot 0 is shifted out by the first step
      const int tt = t0 - K + k;
      Vec16<T> xv;
      if (tt >= 0) {
        xv.load(x + (rx + tt) * ld_x + d0);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) xv.v[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < V; ++i) win.xs[k][i] = xv.v[i];
    }
    // one step t: g[t] = d_u[t] SiLU'(conv[t]) (zero past the end); the weight
    // and bias sums if the chunk owns t; d_x[t - (K-1)] once its window is full
    const auto step = [&](int t, const Vec16<T>& xv, const Vec16<T>& uv, bool valid, bool own) {
      float cv[V];
      win.push_x(xv, cv);
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const float s = sigmoid(cv[i]);
        const float g = valid ? uv.v[i] * s * (1.f + cv[i] * (1.f - s)) : 0.f;
#pragma unroll
        for (int k = 0; k + 1 < K; ++k) win.gs[k][i] = win.gs[k + 1][i];
        win.gs[K - 1][i] = g;
        if (own) {
#pragma unroll
          for (int k = 0; k < K; ++k) dw[k][i] = fmaf(g, win.xs[k][i], dw[k][i]);
          dw[K][i] += g;
        }
      }
      const int to = t - (K - 1);
      if (to >= t0) {
        Vec16<T> o;
#pragma unroll
        for (int i = 0; i < V; ++i) {
          float acc = 0.f;
#pragma unroll
          for (int k = 0; k < K; ++k) acc = fmaf(win.gs[K - 1 - k][i], win.wk[k][i], acc);
          o.v[i] = acc;
        }
        o.store(d_x + (rx + to) * ld_dx + d0);
      }
    };
    // steps t0 .. t1 + K - 2 in groups of kConvLoad; the rows of the next group
    // are loaded (raw) before the current group runs.  Rows are clamped to the
    // last one the wave reads, so every load is in bounds and unconditional.
    const int te = t1 + K - 1, tlast = min(te, Tn) - 1;
    uint4 xr[kConvLoad], ur[kConvLoad];
#pragma unroll
    for (int s = 0; s < kConvLoad; ++s) {
      const int t = min(t0 + s, tlast);
      xr[s] = *reinterpret_cast<const uint4*>(x + (rx + t) * ld_x + d0);
      ur[s] = *reinterpret_cast<const uint4*>(d_u + (rx + t) * ld_du + d0);
    }
    for (int tb = t0; tb < te; tb += kConvLoad) {
      uint4 xn[kConvLoad], un[kConvLoad];
#pragma unroll
      for (int s = 0; s < kConvLoad; ++s) {
        const int t = min(tb + kConvLoad + s, tlast);
        xn[s] = *reinterpret_cast<const uint4*>(x + (rx + t) * ld_x + d0);
        un[s] = *reinterpret_cast<const uint4*>(d_u + (rx + t) * ld_du + d0);
      }
#pragma unroll
      for (int s = 0; s < kConvLoad; ++s) {
        const int t = tb + s;
        if (t < te) {
          Vec16<T> xv, uv;
          xv.set(xr[s]);
          uv.set(ur[s]);
          step(t, xv, uv, t < Tn, t < t1);
        }
        xr[s] = xn[s];
        ur[s] = un[s];
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int k = 0; k <= K; ++k)
#pragma unroll
      for (int i = 0; i < V; ++i) red[wave - 1][k * V + i][lane] = dw[k][i];
  }
  __syncthreads();
  if (wave == 0 && on) {
    float* dst = part + (((size_t)blockIdx.z * gridDim.y + blockIdx.y) * (K + 1)) * Di + d0;
#pragma unroll
    for (int k = 0; k <= K; ++k) {
#pragma unroll
      for (int i = 0; i < V; i += 4) {
        float4 o;
        o.x = dw[k][i] + red[0][k * V + i][lane] + red[1][k * V + i][lane] + red[2][k * V + i][lane];
        o.y = dw[k][i + 1] + red[0][k * V + i + 1][lane] + red[1][k * V + i + 1][lane] + red[2][k * V + i + 1][lane];
        o.z = dw[k][i + 2] + red[0][k * V + i + 2][lane] + red[1][k * V + i + 2][lane] + red[2][k * V + i + 2][lane];
        o.w = dw[k][i + 3] + red[0][k * V + i + 3][lane] + red[1][k * V + i + 3][lane] + red[2][k * V + i + 3][lane];
        *reinterpret_cast<float4*>(dst + (size_t)k * Di + i) = o;
      }
    }
  }
}

// d_w[d, k] and d_bias[d]: sums over the parts [parts][K + 1][Di] in a fixed
// order; a block owns 64 of the (K + 1) Di columns, its four waves take every
// fourth part and combine in LDS
template <int K>
__global__ __launch_bounds__(kPwBlock) void conv1d_bwd_finalize(const float* __restrict__ part,
                                                                float* __restrict__ d_w,
                                                                float* __restrict__ d_bias, int parts, int Di,
                                                                int accumulate) {
  __shared__ float s[4][kWave];
  const int lane = threadIdx.x & (kWave - 1), grp = threadIdx.x / kWave;
  const int ncol = (K + 1) * Di;
  const int col = blockIdx.x * kWave + lane;
  float acc = 0.f;
  if (col < ncol) {
#pragma unroll 8
    for (int p = grp; p < parts; p += 4) acc += part[(size_t)p * ncol + col];
  }
  s[grp][lane] = acc;
  __syncthreads();
  if (grp == 0 && col < ncol) {
    const float v = s[0][lane] + s[1][lane] + s[2][lane] + s[3][lane];
    const int k = col / Di, d = col - k * Di;
    float* dst = k < K ? &d_w[(size_t)d * K + k] : d_bias ? &d_bias[d] : nullptr;
    if (dst) *dst = accumulate ? *dst + v : v;
  }
}

// ---------------------------------------------------------------------------
// rmsnorm: a block takes kRmsRows rows; each thread owns columns tid + 256 j.
constexpr int kRmsRows = 32;
constexpr int kRmsMaxCols = 16;  // dim <= 4096

__device__ __forceinline__ float2 block_sum2(float2 v, float2* sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    v.x += __shfl_xor(v.x, o);
    v.y += __shfl_xor(v.y, o);
  }
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  float2 r = make_float2(0.f, 0.f);
#pragma unroll
  for (int w = 0; w < kPwBlock / kWave; ++w) {
    r.x += sh[w].x;
    r.y += sh[w].y;
  }
  return r;
}

template <typename T>
__global__ __launch_bounds__(kPwBlock) void rmsnorm_bwd_kernel(
    const T* __restrict__ x, const float* __restrict__ w, const T* __restrict__ dy, const T* __restrict__ dres,
    T* __restrict__ dx, float* __restrict__ part, int64_t rows, int dim, float eps) {
  __shared__ float2 red[kPwBlock / kWave];
  const int tid = threadIdx.x;
  const int ncol = (dim + kPwBlock - 1) / kPwBlock;
  float wv[kRmsMaxCols], dw[kRmsMaxCols];
#pragma unroll
  for (int j = 0; j < kRmsMaxCols; ++j) {
    const int col = tid + j * kPwBlock;
    wv[j] = (j < ncol && col < dim) ? w[col] : 0.f;
    dw[j] = 0.f;
  }
  const int64_t r0 = (int64_t)blockIdx.x * kRmsRows;
  const int64_t r1 = min(rows, r0 + kRmsRows);
  const float inv_dim = 1.f / (float)dim;
  for (int64_t r = r0; r < r1; ++r) {
    float xv[kRmsMaxCols], gv[kRmsMaxCols];
    float2 acc = make_float2(0.f, 0.f);
#pragma unroll
    for (int j = 0; j < kRmsMaxCols; ++j) {
      const int col = tid + j * kPwBlock;
      const bool ok = j < ncol && col < dim;
      xv[j] = ok ? ld(x, (size_t)r * dim + col) : 0.f;
      gv[j] = ok ? ld(dy, (size_t)r * dim + col) : 0.f;
      acc.x = fmaf(xv[j], xv[j], acc.x);
      acc.y = fmaf(gv[j] * wv[j], xv[j], acc.y);
    }
    const float2 sums = block_sum2(acc, red);
    const float inv_r = 1.f / sqrtf(sums.x * inv_dim + eps);
    const float dot = sums.y * inv_dim;
    const float c3 = inv_r * inv_r * inv_r * dot;
#pragma unroll
    for (int j = 0; j < kRmsMaxCols; ++j) {
      const int col = tid + j * kPwBlock;
      if (j < ncol && col < dim) {
        float v = inv_r * wv[j] * gv[j] - c3 * xv[j];
        if (dres) v += ld(dres, (size_t)r * dim + col);
        st(dx, (size_t)r * dim + col, v);
        dw[j] = fmaf(gv[j] * xv[j], inv_r, dw[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kRmsMaxCols; ++j) {
    const int col = tid + j * kPwBlock;
    if (j < ncol && col < dim) part[(size_t)blockIdx.x * dim + col] = dw[j];
  }
}

// Wave-per-row RMSNorm for rows whose length is a multiple of the 16-byte
// vector (8 bf16 / 4 float) and at most 64 * VEC * kRmsMaxVec: each lane holds
// vectors lane + 64 j of the row, the two row sums reduce inside the wave, and
// the weight-gradient sums stay in registers over the block's rows before the
// four waves combine them in LDS.
constexpr int kRmsMaxVec = 6;
// rows per wave of the wave-per-row kernels: a wave loads the weight row once
// (as float, twice the bytes of a bf16 input row) for all its rows, while enough
// blocks remain for several waves per SIMD to hide each row's load -> row sum ->
// store chain; on the layer's [16384, 1536] bf16 rows 4 (forward) and 8
// (backward) measured faster than 1 / 2, 2 / 4 and 8 / 16
constexpr int kRmsFwdWaveRows = 4;
constexpr int kRmsBwdWaveRows = 8;  // also sets the number of weight-sum partials

template <typename T, int J>
__global__ __launch_bounds__(kPwBlock) void rmsnorm_fwd_wave(const T* __restrict__ x, const float* __restrict__ w,
                                                             T* __restrict__ xn, int64_t rows, int dim, float eps) {
  constexpr int V = Vec16<T>::N;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nvec = dim / V;
  float wv[J][V];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = (lane + kWave * j) * V;
#pragma unroll
    for (int i = 0; i < V; ++i) wv[j][i] = (lane + kWave * j < nvec) ? w[c + i] : 0.f;
  }
  const float inv_dim = 1.f / (float)dim;
  const int64_t r0 = (int64_t)blockIdx.x * 4 * kRmsFwdWaveRows, r1 = min(rows, r0 + 4 * kRmsFwdWaveRows);
  // all of the wave's rows are loaded (as raw 16-byte words) before the first
  // is reduced, so their memory latencies overlap
  uint4 raw[kRmsFwdWaveRows][J];
#pragma unroll
  for (int q = 0; q < kRmsFwdWaveRows; ++q) {
    const int64_t r = r0 + wave + 4 * q;
#pragma unroll
    for (int j = 0; j < J; ++j)
      raw[q][j] = (r < r1 && lane + kWave * j < nvec)
                      ? *reinterpret_cast<const uint4*>(x + r * dim + (lane + kWave * j) * V)
                      : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int q = 0; q < kRmsFwdWaveRows; ++q) {
    const int64_t r = r0 + wave + 4 * q;
    if (r >= r1) break;
    Vec16<T> xv[J];
    float ss[1] = {0.f};
#pragma unroll
    for (int j = 0; j < J; ++j) {
      xv[j].set(raw[q][j]);
#pragma unroll
      for (int i = 0; i < V; ++i) ss[0] = fmaf(xv[j].v[i], xv[j].v[i], ss[0]);
    }
    wave_reduce_scatter<1>(ss, lane);  // the row's sum of squares in every lane
    const float inv_r = 1.f / sqrtf(ss[0] * inv_dim + eps);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (lane + kWave * j < nvec) {
#pragma unroll
        for (int i = 0; i < V; ++i) xv[j].v[i] = xv[j].v[i] * inv_r * wv[j][i];
        xv[j].store(xn + r * dim + (lane + kWave * j) * V);
      }
    }
  }
}

template <typename T, int J>
__global__ __launch_bounds__(kPwBlock) void rmsnorm_bwd_wave(const T* __restrict__ x, const float* __restrict__ w,
                                                             const T* __restrict__ dy, const T* __restrict__ dres,
                                                             T* __restrict__ dx, float* __restrict__ part,
                                                             int64_t rows, int dim, float eps) {
  constexpr int V = Vec16<T>::N;
  __shared__ float red[4][J * V * kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nvec = dim / V;
  float wv[J][V], dw[J][V];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = (lane + kWave * j) * V;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      wv[j][i] = (lane + kWave * j < nvec) ? w[c + i] : 0.f;
      dw[j][i] = 0.f;
    }
  }
  const float inv_dim = 1.f / (float)dim;
  const int64_t r0 = (int64_t)blockIdx.x * 4 * kRmsBwdWaveRows, r1 = min(rows, r0 + 4 * kRmsBwdWaveRows);
  for (int64_t r = r0 + wave; r < r1; r += 4) {
    Vec16<T> xv[J], gv[J], res[J];
    float ss = 0.f, sd = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (lane + kWave * j < nvec) {
        xv[j].load(x + r * dim + (lane + kWave * j) * V);
        gv[j].load(dy + r * dim + (lane + kWave * j) * V);
        if (dres) res[j].load(dres + r * dim + (lane + kWave * j) * V);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) xv[j].v[i] = gv[j].v[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < V; ++i) {
        ss = fmaf(xv[j].v[i], xv[j].v[i], ss);
        sd = fmaf(gv[j].v[i] * wv[j][i], xv[j].v[i], sd);
      }
    }
    const float inv_r = 1.f / sqrtf(wave_sum(ss) * inv_dim + eps);
    const float c3 = inv_r * inv_r * inv_r * (wave_sum(sd) * inv_dim);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (lane + kWave * j < nvec) {
        Vec16<T> o;
#pragma unroll
        for (int i = 0; i < V; ++i) {
          o.v[i] = inv_r * wv[j][i] * gv[j].v[i] - c3 * xv[j].v[i] + (dres ? res[j].v[i] : 0.f);
          dw[j][i] = fmaf(gv[j].v[i] * xv[j].v[i], inv_r, dw[j][i]);
        }
        o.store(dx + r * dim + (lane + kWave * j) * V);
      }
    }
  }
  // combine the four waves' column sums in a fixed order
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int i = 0; i < V; ++i) red[wave][(j * V + i) * kWave + lane] = dw[j][i];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (lane + kWave * j < nvec) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const int k = (j * V + i) * kWave + lane;
          part[(size_t)blockIdx.x * dim + (lane + kWave * j) * V + i] = red[0][k] + red[1][k] + red[2][k] + red[3][k];
        }
      }
    }
  }
}

// dw[col] = sum over parts, in a fixed order: a block owns 64 columns, its four
// waves take every fourth part and combine in LDS
__global__ __launch_bounds__(kPwBlock) void rmsnorm_bwd_finalize(const float* __restrict__ part,
                                                                 float* __restrict__ dw, int parts, int dim,
                                                                 int accumulate) {
  __shared__ float s[4][kWave];
  const int lane = threadIdx.x & (kWave - 1), grp = threadIdx.x / kWave;
  const int col = blockIdx.x * kWave + lane;
  float acc = 0.f;
  if (col < dim) {
#pragma unroll 8
    for (int p = grp; p < parts; p += 4) acc += part[(size_t)p * dim + col];
  }
  s[grp][lane] = acc;
  __syncthreads();
  if (grp == 0 && col < dim) {
    const float v = s[0][lane] + s[1][lane] + s[2][lane] + s[3][lane];
    dw[col] = accumulate ? dw[col] + v : v;
  }
}

// ---------------------------------------------------------------------------
// forward pieces (bf16 storage, float arithmetic)

// xn = x * w / sqrt(mean(x^2) + eps), rows of `dim` <= 4096
__global__ __launch_bounds__(kPwBlock) void rmsnorm_fwd_kernel(const bf16* __restrict__ x, const float* __restrict__ w,
                                                               bf16* __restrict__ xn, int64_t rows, int dim,
                                                               float eps) {
  __shared__ float2 red[kPwBlock / kWave];
  const int tid = threadIdx.x;
  const int ncol = (dim + kPwBlock - 1) / kPwBlock;
  const int64_t r0 = (int64_t)blockIdx.x * kRmsRows;
  const int64_t r1 = min(rows, r0 + kRmsRows);
  const float inv_dim = 1.f / (float)dim;
  for (int64_t r = r0; r < r1; ++r) {
    float xv[kRmsMaxCols];
    float2 acc = make_float2(0.f, 0.f);
#pragma unroll
    for (int j = 0; j < kRmsMaxCols; ++j) {
      const int col = tid + j * kPwBlock;
      xv[j] = (j < ncol && col < dim) ? ld(x, (size_t)r * dim + col) : 0.f;
      acc.x = fmaf(xv[j], xv[j], acc.x);
    }
    const float inv_r = 1.f / sqrtf(block_sum2(acc, red).x * inv_dim + eps);
#pragma unroll
    for (int j = 0; j < kRmsMaxCols; ++j) {
      const int col = tid + j * kPwBlock;
      if (j < ncol && col < dim) st(xn, (size_t)r * dim + col, xv[j] * inv_r * w[col]);
    }
  }
}

// u[b,t,d] = SiLU(bias[d] + sum_k w[d,k] x[b, t-(K-1)+k, d]), on 8-channel
// vectors: a lane per vector and a wave per chunk of tv steps, as in the
// vector conv backward
template <int K>
__global__ __launch_bounds__(kPwBlock) void conv_silu_fwd_vec(const bf16* __restrict__ x, int ld_x,
                                                              const float* __restrict__ w,
                                                              const float* __restrict__ bias, bf16* __restrict__ u,
                                                              int ld_u, int Tn, int Di, int tv) {
  constexpr int V = Vec16<bf16>::N;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int d0 = (blockIdx.x * kWave + lane) * V;
  const int t0 = (blockIdx.y * kConvWaves + wave) * tv;
  if (d0 >= Di || t0 >= Tn) return;
  const int t1 = min(Tn, t0 + tv);
  const size_t rx = (size_t)blockIdx.z * Tn;
  ConvWindow<bf16, K> win;
  win.init(w, bias, d0);
#pragma unroll
  for (int k = 1; k < K; ++k) {
    const int tt = t0 - K + k;
    Vec16<bf16> xv;
    if (tt >= 0) {
      xv.load(x + (rx + tt) * ld_x + d0);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) xv.v[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < V; ++i) win.xs[k][i] = xv.v[i];
  }
  uint4 xr[kConvLoad];
#pragma unroll
  for (int s = 0; s < kConvLoad; ++s)
    xr[s] = *reinterpret_cast<const uint4*>(x + (rx + min(t0 + s, t1 - 1)) * ld_x + d0);
  for (int tb = t0; tb < t1; tb += kConvLoad) {
    uint4 xn[kConvLoad];
#pragma unroll
    for (int s = 0; s < kConvLoad; ++s)
      xn[s] = *reinterpret_cast<const uint4*>(x + (rx + min(tb + kConvLoad + s, t1 - 1)) * ld_x + d0);
#pragma unroll
    for (int s = 0; s < kConvLoad; ++s) {
      if (tb + s < t1) {
        Vec16<bf16> xv;
        xv.set(xr[s]);
        float cv[V];
        win.push_x(xv, cv);
        Vec16<bf16> o;
#pragma unroll
        for (int i = 0; i < V; ++i) o.v[i] = cv[i] * sigmoid(cv[i]);
        o.store(u + (rx + tb + s) * ld_u + d0);
      }
      xr[s] = xn[s];
    }
  }
}

// gated = y * SiLU(z) on 8-channel vectors, z rows of stride ld_z
__global__ __launch_bounds__(kPwBlock) void gate_fwd_vec(const bf16* __restrict__ y, const bf16* __restrict__ z,
                                                         int ld_z, bf16* __restrict__ g, int64_t rows, int nvec) {
  constexpr int V = Vec16<bf16>::N;
  const int64_t n = rows * nvec;
  const int64_t stride = (int64_t)gridDim.x * kPwBlock;
  for (int64_t i = (int64_t)blockIdx.x * kPwBlock + threadIdx.x; i < n; i += stride) {
    const int64_t r = i / nvec;
    const int dv = (int)(i - r * nvec);
    Vec16<bf16> yv, zv;
    yv.load(y + i * V);
    zv.load(z + (size_t)r * ld_z + (size_t)dv * V);
#pragma unroll
    for (int k = 0; k < V; ++k) yv.v[k] = yv.v[k] * zv.v[k] * sigmoid(zv.v[k]);
    yv.store(g + i * V);
  }
}

// delta = softplus(v + b) with v > 20 passed through, in place on [rows, Di] bf16,
// 8 channels per lane.  softplus(x) = max(x, 0) + log(1 + e^-|x|) on the
// hardware exp2 / log2; below 2^-10 log(1 + y) is taken as y (1 - y / 2),
// where 1 + y would drop y's low digits (relative error under 1e-6 either
// way, far below bf16's 2^-9).
__device__ __forceinline__ float softplus_f(float x) {
  if (x > 20.f) return x;
  const float y = fast_exp2(-fabsf(x) * kLog2e);
  const float l = y < 0.0009765625f ? y * (1.f - 0.5f * y) : __builtin_amdgcn_logf(1.f + y) * kLn2;
  return fmaxf(x, 0.f) + l;
}

__global__ __launch_bounds__(kPwBlock) void bias_softplus_kernel(bf16* __restrict__ v, const float* __restrict__ b,
                                                                 int64_t rows, int Di) {
  const int64_t n = rows * Di;
  const int64_t stride = (int64_t)gridDim.x * kPwBlock;
  for (int64_t i = (int64_t)blockIdx.x * kPwBlock + threadIdx.x; i < n; i += stride)
    st(v, i, softplus_f(ld(v, i) + b[i % Di]));
}

__global__ __launch_bounds__(kPwBlock) void bias_softplus_vec(bf16* __restrict__ v, const float* __restrict__ b,
                                                              int64_t rows, int nvec) {
  constexpr int V = Vec16<bf16>::N;
  const int64_t n = rows * nvec;
  const int64_t stride = (int64_t)gridDim.x * kPwBlock;
  for (int64_t i = (int64_t)blockIdx.x * kPwBlock + threadIdx.x; i < n; i += stride) {
    const int dv = (int)(i % nvec);
    Vec16<bf16> x;
    x.load(v + i * V);
    float bb[V];
    if (b) {  // the bias row is 16-byte aligned (checked by the launcher)
      const float4 b0 = reinterpret_cast<const float4*>(b)[2 * dv], b1 = reinterpret_cast<const float4*>(b)[2 * dv + 1];
      bb[0] = b0.x; bb[1] = b0.y; bb[2] = b0.z; bb[3] = b0.w; bb[4] = b1.x; bb[5] = b1.y; bb[6] = b1.z; bb[7] = b1.w;
    } else {
#pragma unroll
      for (int k = 0; k < V; ++k) bb[k] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < V; ++k) x.v[k] = softplus_f(x.v[k] + bb[k]);
    x.store(v + i * V);
  }
}

// y[r, c] += b[c] on bf16 rows of n (a linear layer's bias)
__global__ __launch_bounds__(kPwBlock) void bias_add_kernel(bf16* __restrict__ y, const float* __restrict__ b,
                                                            int64_t rows, int n) {
  const int64_t total = rows * n;
  const int64_t stride = (int64_t)gridDim.x * kPwBlock;
  for (int64_t i = (int64_t)blockIdx.x * kPwBlock + threadIdx.x; i < total; i += stride)
    st(y, i, ld(y, i) + b[(int)(i % n)]);
}

namespace {
int grid_for(int64_t n) {
  const int64_t want = (n + kPwBlock - 1) / kPwBlock;
  return (int)(want < 8192 ? want : 8192);
}
}  // namespace

void launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n > 0) hipLaunchKernelGGL(fill_zero_f32, dim3((unsigned)((n + kPwBlock - 1) / kPwBlock)), dim3(kPwBlock), 0, st, p, n);
}

// vectors of 16 bytes per lane the wave-per-row kernels need for a row, 0 if they do not apply
template <typename T>
int rms_wave_vecs(const void* a, const void* b, const void* c, const void* d, int dim) {
  constexpr int V = 16 / sizeof(T);
  const auto al = [](const void* p) { return p == nullptr || aligned16(p); };
  if (dim % V != 0 || !al(a) || !al(b) || !al(c) || !al(d)) return 0;
  const int j = (dim / V + kWave - 1) / kWave;
  return j <= kRmsMaxVec ? j : 0;
}

void launch_rmsnorm_fwd(const bf16* x, const float* w, bf16* xn, int64_t rows, int dim, float eps, hipStream_t st) {
  if (rows == 0) return;
  const int j = rms_wave_vecs<bf16>(x, xn, nullptr, nullptr, dim);
  const dim3 grid((unsigned)((rows + 4 * kRmsFwdWaveRows - 1) / (4 * kRmsFwdWaveRows)));
  switch (j) {
#define RMS_FWD(J) \
  case J: hipLaunchKernelGGL((rmsnorm_fwd_wave<bf16, J>), grid, dim3(kPwBlock), 0, st, x, w, xn, rows, dim, eps); return;
    RMS_FWD(1) RMS_FWD(2) RMS_FWD(3) RMS_FWD(4) RMS_FWD(5) RMS_FWD(6)
#undef RMS_FWD
    default:
      hipLaunchKernelGGL(rmsnorm_fwd_kernel, dim3((unsigned)((rows + kRmsRows - 1) / kRmsRows)), dim3(kPwBlock), 0,
                         st, x, w, xn, rows, dim, eps);
  }
}

void launch_conv_silu_fwd(const bf16* x, int ld_x, const float* w, const float* bias, bf16* u, int ld_u, int Bt,
                          int Tn, int Di, int K, hipStream_t st) {
  if ((int64_t)Bt * Tn == 0) return;
  const int nx = (Di / 8 + kWave - 1) / kWave;
  const int tv = conv_steps_per_wave(Tn, nx, Bt, K, kConvFwdBlocksPerCU);
  const dim3 grid(nx, (Tn + kConvWaves * tv - 1) / (kConvWaves * tv), Bt);
#define CONV_FWD(KV)                                                                                              \
  case KV:                                                                                                        \
    hipLaunchKernelGGL(conv_silu_fwd_vec<KV>, grid, dim3(kPwBlock), 0, st, x, ld_x, w, bias, u, ld_u, Tn, Di, tv); \
    break;
  switch (K) { CONV_FWD(1) CONV_FWD(2) CONV_FWD(3) CONV_FWD(4) CONV_FWD(5) CONV_FWD(6) CONV_FWD(7) CONV_FWD(8) }
#undef CONV_FWD
}

void launch_gate_fwd(const bf16* y, const bf16* z, int ld_z, bf16* g, int64_t rows, int Di, hipStream_t st) {
  if (rows * Di == 0) return;
  hipLaunchKernelGGL(gate_fwd_vec, dim3(grid_for(rows * Di / 8)), dim3(kPwBlock), 0, st, y, z, ld_z, g, rows, Di / 8);
}

void launch_bias_add(bf16* y, const float* b, int64_t rows, int n, hipStream_t st) {
  if (rows * n == 0) return;
  hipLaunchKernelGGL(bias_add_kernel, dim3(grid_for(rows * n)), dim3(kPwBlock), 0, st, y, b, rows, n);
}

void launch_bias_softplus(bf16* v, const float* b, int64_t rows, int Di, hipStream_t st) {
  if (rows * Di == 0) return;
  if (b && !aligned16(b)) {  // a bias that is not 16-byte aligned: one element per thread
    hipLaunchKernelGGL(bias_softplus_kernel, dim3(grid_for(rows * Di)), dim3(kPwBlock), 0, st, v, b, rows, Di);
    return;
  }
  hipLaunchKernelGGL(bias_softplus_vec, dim3(grid_for(rows * Di / 8)), dim3(kPwBlock), 0, st, v, b, rows, Di / 8);
}

}  // namespace ssm

using namespace ssm;

extern "C" int gating_bwd(const void* d_out, const void* y, const void* z, void* d_y, void* d_z, int64_t n,
                          int dtype, void* stream) {
  if (n < 0) return fail(SSM_ERR_INVALID_ARG, "n = %lld", (long long)n);
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (n == 0) return SSM_OK;
  if (!d_out || !y || !z || !d_y || !d_z) return fail(SSM_ERR_INVALID_ARG, "a tensor pointer is null");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t want = (n + kPwBlock - 1) / kPwBlock;
  const int blocks = (int)(want < 8192 ? want : 8192);
  if (dtype == SSM_F32)
    hipLaunchKernelGGL(gating_bwd_kernel<float>, dim3(blocks), dim3(kPwBlock), 0, st, (const float*)d_out,
                       (const float*)y, (const float*)z, (float*)d_y, (float*)d_z, n);
  else
    hipLaunchKernelGGL(gating_bwd_kernel<bf16>, dim3(blocks), dim3(kPwBlock), 0, st, (const bf16*)d_out,
                       (const bf16*)y, (const bf16*)z, (bf16*)d_y, (bf16*)d_z, n);
  return check_launch("gating_bwd");
}

extern "C" size_t conv1d_bwd_workspace_size(int batch, int seqlen, int d_inner, int d_conv) {
  if (batch <= 0 || seqlen <= 0 || d_inner <= 0 || d_conv <= 0 || d_conv > kMaxTaps) return 0;
  const size_t nchunk = (seqlen + kConvT - 1) / kConvT;
  return align_up((size_t)batch * nchunk * (d_conv + 1) * d_inner * sizeof(float));
}

extern "C" int conv1d_bwd(const void* x, const float* w, const float* bias, const void* d_u, void* d_x, float* d_w,
                          float* d_bias, int batch, int seqlen, int d_inner, int d_conv, int ld_x, int ld_du,
                          int ld_dx, int flags, void* workspace, size_t ws_bytes, int dtype, void* stream) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (flags & ~SSM_BWD_ACCUMULATE) return fail(SSM_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  const int acc = (flags & SSM_BWD_ACCUMULATE) ? 1 : 0;
  if (batch < 0 || seqlen < 0 || d_inner <= 0 || d_conv <= 0)
    return fail(SSM_ERR_INVALID_ARG, "bad size (batch %d seqlen %d d_inner %d d_conv %d)", batch, seqlen, d_inner,
                d_conv);
  if (d_conv > kMaxTaps) return fail(SSM_ERR_UNSUPPORTED, "d_conv %d > %d", d_conv, kMaxTaps);
  if (ld_x < d_inner || ld_du < d_inner || ld_dx < d_inner)
    return fail(SSM_ERR_INVALID_ARG, "row strides below d_inner");
  if (!w || !d_w) return fail(SSM_ERR_INVALID_ARG, "w and d_w are required");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((size_t)batch * seqlen == 0) {  // sums over nothing
    if (acc) return SSM_OK;
    hipLaunchKernelGGL(fill_zero_f32, dim3((d_inner * d_conv + kPwBlock - 1) / kPwBlock), dim3(kPwBlock), 0, st,
                       d_w, (int64_t)d_inner * d_conv);
    if (d_bias)
      hipLaunchKernelGGL(fill_zero_f32, dim3((d_inner + kPwBlock - 1) / kPwBlock), dim3(kPwBlock), 0, st, d_bias,
                         (int64_t)d_inner);
    return check_launch("conv1d_bwd (empty)");
  }
  if (!x || !d_u || !d_x) return fail(SSM_ERR_INVALID_ARG, "a tensor pointer is null");
  const size_t need = conv1d_bwd_workspace_size(batch, seqlen, d_inner, d_conv);
  if (!workspace || ws_bytes < need || !aligned256(workspace))
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed (256-byte aligned)",
                workspace ? ws_bytes : 0, need);
  float* part = static_cast<float*>(workspace);
  const int V = dtype == SSM_F32 ? 4 : 8;
  const bool vec = d_inner % V == 0 && ld_x % V == 0 && ld_du % V == 0 && ld_dx % V == 0 && aligned16(x) &&
                   aligned16(d_u) && aligned16(d_x) && aligned16(workspace);
  const int nx = vec ? (d_inner / V + kWave - 1) / kWave : (d_inner + kPwBlock - 1) / kPwBlock;
  const int tv = vec ? conv_steps_per_wave(seqlen, nx, batch, d_conv, kConvBwdBlocksPerCU) : 0;
  const int nchunk = vec ? (seqlen + kConvWaves * tv - 1) / (kConvWaves * tv) : (seqlen + kConvT - 1) / kConvT;
  const dim3 grid(nx, nchunk, batch);
  const dim3 fgrid(((d_conv + 1) * d_inner + kWave - 1) / kWave);
#define CONV_CASE(TY, KV)                                                                                      \
  case KV:                                                                                                     \
    if (vec)                                                                                                   \
      hipLaunchKernelGGL((conv1d_bwd_vec<TY, KV>), grid, dim3(kPwBlock), 0, st, (const TY*)x, w, bias,        \
                         (const TY*)d_u, (TY*)d_x, part, seqlen, d_inner, ld_x, ld_du, ld_dx, tv);            \
    else                                                                                                       \
      hipLaunchKernelGGL((conv1d_bwd_kernel<TY, KV>), grid, dim3(kPwBlock), 0, st, (const TY*)x, w, bias,     \
                         (const TY*)d_u, (TY*)d_x, part, batch, seqlen, d_inner, ld_x, ld_du, ld_dx, nchunk); \
    hipLaunchKernelGGL((conv1d_bwd_finalize<KV>), fgrid, dim3(kPwBlock), 0, st, part, d_w, d_bias,            \
                       batch * nchunk, d_inner, acc);                                                         \
    break;
  if (dtype == SSM_F32) {
    switch (d_conv) { CONV_CASE(float, 1) CONV_CASE(float, 2) CONV_CASE(float, 3) CONV_CASE(float, 4)
                      CONV_CASE(float, 5) CONV_CASE(float, 6) CONV_CASE(float, 7) CONV_CASE(float, 8) }
  } else {
    switch (d_conv) { CONV_CASE(bf16, 1) CONV_CASE(bf16, 2) CONV_CASE(bf16, 3) CONV_CASE(bf16, 4)
                      CONV_CASE(bf16, 5) CONV_CASE(bf16, 6) CONV_CASE(bf16, 7) CONV_CASE(bf16, 8) }
  }
#undef CONV_CASE
  return check_launch("conv1d_bwd");
}

extern "C" size_t rmsnorm_bwd_workspace_size(int64_t rows, int dim) {
  if (rows <= 0 || dim <= 0 || dim > kPwBlock * kRmsMaxCols) return 0;
  // one partial row per block of either kernel
  constexpr int rows_per_block = kRmsRows < 4 * kRmsBwdWaveRows ? kRmsRows : 4 * kRmsBwdWaveRows;
  const size_t blocks = (size_t)((rows + rows_per_block - 1) / rows_per_block);
  return align_up(blocks * dim * sizeof(float));
}

extern "C" int rmsnorm_bwd(const void* x, const float* w, const void* dy, const void* d_residual, void* dx,
                           float* dw, int64_t rows, int dim, float eps, int flags, void* workspace, size_t ws_bytes,
                           int dtype, void* stream) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (flags & ~SSM_BWD_ACCUMULATE) return fail(SSM_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  const int acc = (flags & SSM_BWD_ACCUMULATE) ? 1 : 0;
  if (rows < 0 || dim <= 0) return fail(SSM_ERR_INVALID_ARG, "bad size (rows %lld dim %d)", (long long)rows, dim);
  if (dim > kPwBlock * kRmsMaxCols) return fail(SSM_ERR_UNSUPPORTED, "dim %d > %d", dim, kPwBlock * kRmsMaxCols);
  if (!(eps >= 0.f)) return fail(SSM_ERR_INVALID_ARG, "eps must be >= 0");
  if (!dw) return fail(SSM_ERR_INVALID_ARG, "dw is required");
  if (rows == 0) {  // sum over no rows
    if (acc) return SSM_OK;
    hipLaunchKernelGGL(fill_zero_f32, dim3((dim + kPwBlock - 1) / kPwBlock), dim3(kPwBlock), 0,
                       static_cast<hipStream_t>(stream), dw, (int64_t)dim);
    return check_launch("rmsnorm_bwd (empty)");
  }
  if (!x || !w || !dy || !dx) return fail(SSM_ERR_INVALID_ARG, "a tensor pointer is null");
  const size_t need = rmsnorm_bwd_workspace_size(rows, dim);
  if (!workspace || ws_bytes < need || !aligned256(workspace))
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed (256-byte aligned)",
                workspace ? ws_bytes : 0, need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(workspace);
  int blocks = 0;
  const int jw = dtype == SSM_F32 ? rms_wave_vecs<float>(x, dy, d_residual, dx, dim)
                                  : rms_wave_vecs<bf16>(x, dy, d_residual, dx, dim);
  if (jw > 0) {
    blocks = (int)((rows + 4 * kRmsBwdWaveRows - 1) / (4 * kRmsBwdWaveRows));
#define RMS_BWD(TY, J)                                                                                          \
  case J:                                                                                                       \
    hipLaunchKernelGGL((rmsnorm_bwd_wave<TY, J>), dim3(blocks), dim3(kPwBlock), 0, st, (const TY*)x, w,         \
                       (const TY*)dy, (const TY*)d_residual, (TY*)dx, part, rows, dim, eps);                   \
    break;
    if (dtype == SSM_F32) {
      switch (jw) { RMS_BWD(float, 1) RMS_BWD(float, 2) RMS_BWD(float, 3) RMS_BWD(float, 4) RMS_BWD(float, 5)
                    RMS_BWD(float, 6) }
    } else {
      switch (jw) { RMS_BWD(bf16, 1) RMS_BWD(bf16, 2) RMS_BWD(bf16, 3) RMS_BWD(bf16, 4) RMS_BWD(bf16, 5)
                    RMS_BWD(bf16, 6) }
    }
#undef RMS_BWD
  } else {
    blocks = (int)((rows + kRmsRows - 1) / kRmsRows);
    if (dtype == SSM_F32)
      hipLaunchKernelGGL(rmsnorm_bwd_kernel<float>, dim3(blocks), dim3(kPwBlock), 0, st, (const float*)x, w,
                         (const float*)dy, (const float*)d_residual, (float*)dx, part, rows, dim, eps);
    else
      hipLaunchKernelGGL(rmsnorm_bwd_kernel<bf16>, dim3(blocks), dim3(kPwBlock), 0, st, (const bf16*)x, w,
                         (const bf16*)dy, (const bf16*)d_residual, (bf16*)dx, part, rows, dim, eps);
  }
  hipLaunchKernelGGL(rmsnorm_bwd_finalize, dim3((dim + kWave - 1) / kWave), dim3(kPwBlock), 0, st, part, dw,
                     blocks, dim, acc);
  return check_launch("rmsnorm_bwd");
}
