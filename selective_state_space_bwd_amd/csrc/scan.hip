// Selective-scan forward and backward for gfx950.
//
// Method (mamba-rs 0.5.1 cpu/backward.rs, Phases B2 and B3): the page walks t
// backwards once, reading three saved per-step state tensors (da_exp, h_prev,
// h_curr, each [T, d_inner*d_state]).  Here nothing per step and per state
// goes to memory.  One lane owns one channel (b, d) and keeps its d_state
// states in registers; B_t and C_t are the same for every lane of a block and
// are read from scalar registers or a block-wide LDS copy.  Time is cut into segments that run in parallel,
// and each segment into chunks of kChunk steps:
//
//   1. summary  (per segment, forward in t): the segment's local states from a
//      zero start, with the state before every chunk written out
//      (checkpoints), the local end state, and the local adjoint summary
//      G = sum_t (prod_{r<=t} a_r) dy_t C_t that the next carry needs.
//   2. carry    (per channel, over segments): the pair operator
//      (a1, v1) + (a2, v2) = (a2 a1, a2 v1 + v2) joins the segments, forward for
//      the state entering each segment and backward for the adjoint leaving it;
//      a segment's decay is exp(A * sum of its delta).
//   3. main     (per segment, chunks in reverse): rebuild the chunk's states
//      from its checkpoint (corrected by the carried-in state), keep a_t h_{t-1}
//      in registers, then walk the chunk backwards with the adjoint g.  d_B and
//      d_C (sums over channels) are reduced inside the wave with permlane swaps
//      and DPP, across the block's waves in LDS, and across blocks as
//      fixed-order partials; d_A_log and d_D (sums over batch and time) are kept
//      per lane over the segment and written as partials.  Float storage runs
//      it one channel per lane, and so does bf16 from given chunk states; bf16
//      rebuilding its states runs on lane pairs that share two channels, each
//      lane holding half the states of both (3').
//   4. finalize: fixed-order sums of the partials.
// Nothing uses atomics, so results are bitwise repeatable.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <type_traits>

#include "common.hpp"

namespace ssm {

constexpr int kChunk = 8;    // steps rebuilt and held in registers at a time
constexpr int kBlock = 256;  // threads (and channels) per block (4 waves)

struct ScanShape {
  int Bt, T, Di, ld_bc, ld_dbc, ld_z;
  int seg, nseg, nchunk, ntile;
};

struct ScanWs {
  float* ckpt;     // [Bt, nchunk, N, Di]  local state before each chunk
  float* ckpt_sd;  // [Bt, nchunk, Di]     sum of delta from the segment start
  float* seg_h;    // [Bt, nseg, N, Di]    local end state, then the state entering the segment
  float* seg_g;    // [Bt, nseg, N, Di]    local adjoint summary, then the adjoint leaving it
  float* seg_sd;   // [Bt, nseg, Di]       sum of delta over the segment
  float* part_bc;  // [ntile, Bt, T, 2N]   per-block sums of d_B | d_C
  float* part_a;   // [Bt, nseg, N+1, Di]  per-segment sums for d_A_log | d_D
};

template <int NS>
__device__ __forceinline__ void load_A2(const float* __restrict__ A_log, int d, float (&A2)[NS]) {
#pragma unroll
  for (int n = 0; n < NS; ++n) A2[n] = -expf(A_log[(size_t)d * NS + n]) * kLog2e;
}

// The B | C rows of one 8-step chunk, staged in LDS for the whole block: thread
// i < 8 * 2N holds element (step i / 2N, column i % 2N), B in columns [0, N)
// and C in [N, 2N).  Steps past the chunk's valid length repeat its last row
// (clamp) so every read stays inside the tensors.
template <typename T, int NS>
__device__ __forceinline__ float bc_element(const T* __restrict__ Bb, const T* __restrict__ Cb, int ld_bc, int tc,
                                            int nv, int tid) {
  const int j = tid / (2 * NS), k = tid - j * (2 * NS);
  if (tid >= kChunk * 2 * NS) return 0.f;
  const size_t row = (size_t)(tc + min(j, nv - 1)) * ld_bc;
  return k < NS ? ld(Bb, row + k) : ld(Cb, row + (k - NS));
}

// One element of a row whose address is the same in every lane of the wave,
// at a 32-bit per-lane element offset (the row pointer is scalar, the lane's
// part a 32-bit byte offset).
template <typename T>
__device__ __forceinline__ float ld_row(const T* __restrict__ row, uint32_t col) {
  return to_f32(*reinterpret_cast<const T*>(reinterpret_cast<const char*>(row) + col * (uint32_t)sizeof(T)));
}
template <typename T>
__device__ __forceinline__ void st_row(T* __restrict__ row, uint32_t col, float v) {
  *reinterpret_cast<T*>(reinterpret_cast<char*>(row) + col * (uint32_t)sizeof(T)) = from_f32<T>(v);
}

template <int NS>
__device__ __forceinline__ void bc_row(const float (&bcs)[kChunk][2 * NS], int j, float (&Bv)[NS], float (&Cv)[NS]) {
  const float4* p = reinterpret_cast<const float4*>(&bcs[j][0]);
#pragma unroll
  for (int q = 0; q < NS / 4; ++q) {
    const float4 b = p[q], c = p[NS / 4 + q];
    Bv[4 * q] = b.x; Bv[4 * q + 1] = b.y; Bv[4 * q + 2] = b.z; Bv[4 * q + 3] = b.w;
    Cv[4 * q] = c.x; Cv[4 * q + 1] = c.y; Cv[4 * q + 2] = c.z; Cv[4 * q + 3] = c.w;
  }
}

// ---------------------------------------------------------------------------
// 1. segment summaries.  BWD adds the chunk checkpoints and the adjoint summary.
//
// Every chunk takes one branch-free path.  Lane offsets are 32-bit from
// per-batch base pointers.
template <typename T, int NS, bool BWD>
__global__ __launch_bounds__(kBlock) void scan_summary(
    const T* __restrict__ u, const T* __restrict__ delta, const float* __restrict__ A_log,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const T* __restrict__ z,
    const T* __restrict__ dout, float* __restrict__ ckpt, float* __restrict__ ckpt_sd,
    float* __restrict__ seg_h, float* __restrict__ seg_g, float* __restrict__ seg_sd, ScanShape sh) {
  const int d = blockIdx.x * kBlock + threadIdx.x;
  const int s = blockIdx.y, b = blockIdx.z;
  const bool active = d < sh.Di;
  const int dc = active ? d : sh.Di - 1;
  const int Di = sh.Di;
  float A2[NS];
  load_A2<NS>(A_log, dc, A2);
  float h[NS], P[NS], G[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) { h[n] = 0.f; P[n] = 1.f; G[n] = 0.f; }
  float sd = 0.f;
  const int t0 = s * sh.seg, t1 = min(sh.T, t0 + sh.seg);
  const size_t bo = (size_t)b * sh.T * Di;
  const T* __restrict__ ub = u + bo;
  const T* __restrict__ db = delta + bo;
  const T* __restrict__ zb = BWD ? z + (size_t)b * sh.T * sh.ld_z : nullptr;
  const T* __restrict__ gb = BWD ? dout + bo : nullptr;
  const T* __restrict__ Bb = Bm + (size_t)b * sh.T * sh.ld_bc;
  const T* __restrict__ Cb = Cm + (size_t)b * sh.T * sh.ld_bc;

  // the first segment's adjoint summary is never used
  const bool need_g = BWD && s > 0;
  // float prefetches the next chunk's channel values and stages B | C in LDS;
  // bf16 prefetches only the next chunk's delta and u, which keeps it at three
  // waves per SIMD (its z and d_out load at the chunk's start, B | C with scalar
  // loads): measured 20 % faster than loading everything at the chunk's start,
  // while the float path's full prefetch costs bf16 its third wave and a quarter
  constexpr bool kPipe = sizeof(T) == 4;
  // per-step channel values of one chunk; a ragged last chunk reads its last
  // step again and zeroes the extra steps' delta, u and dy below: a = 1 there,
  // so the state, P and G pass through unchanged
  struct Raw {
    float dl[kChunk], uu[kChunk], zr[kChunk], gr[kChunk];
  };
  const auto load_du = [&](int tc, Raw& r) {
    const int nv = min(kChunk, t1 - tc);
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const unsigned off = (unsigned)(tc + min(j, nv - 1)) * Di + dc;
      r.dl[j] = ld(db, off);
      r.uu[j] = ld(ub, off);
    }
  };
  const auto load_zg = [&](int tc, Raw& r) {
    const int nv = min(kChunk, t1 - tc);
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const unsigned tj = (unsigned)(tc + min(j, nv - 1));
      r.zr[j] = ld(zb, tj * sh.ld_z + dc);
      r.gr[j] = ld(gb, tj * Di + dc);
    }
  };
  // Each wave stages its own copy of the chunk's B | C rows (kBcPer elements
  // per lane), so no block barrier is needed: one wave's LDS accesses take
  // effect in program order, and the fences around a wave barrier keep the
  // compiler from moving the reads of the next chunk's rows above their stores.
  constexpr int kBcPer = kChunk * 2 * NS / kWave;
  __shared__ __align__(16) float bcs[kBlock / kWave][kChunk][2 * NS];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  float* const mybc = &bcs[wave][0][0];
  const auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  Raw cur;
  load_du(t0, cur);
  if (kPipe) {
    if (need_g) load_zg(t0, cur);
#pragma unroll
    for (int q = 0; q < kBcPer; ++q)
      mybc[lane + kWave * q] = bc_element<T, NS>(Bb, Cb, sh.ld_bc, t0, min(kChunk, t1 - t0), lane + kWave * q);
    wave_sync();
  }
  for (int tc = t0; tc < t1; tc += kChunk) {
    const bool more = tc + kChunk < t1;
    Raw nxt;
    float bc_next[kBcPer];
    if (more) load_du(tc + kChunk, nxt);
    if (kPipe && more) {
      if (need_g) load_zg(tc + kChunk, nxt);
#pragma unroll
      for (int q = 0; q < kBcPer; ++q)
        bc_next[q] = bc_element<T, NS>(Bb, Cb, sh.ld_bc, tc + kChunk, min(kChunk, t1 - tc - kChunk), lane + kWave * q);
    }
    if (BWD && tc > t0 && active) {
      const size_t c = (size_t)b * sh.nchunk + tc / kChunk;
#pragma unroll
      for (int n = 0; n < NS; ++n) ckpt[(c * NS + n) * Di + d] = h[n];
      ckpt_sd[c * Di + d] = sd;
    }
    if (!kPipe && need_g) load_zg(tc, cur);
    const int nv = min(kChunk, t1 - tc);
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const bool ok = j < nv;
      const float dlj = ok ? cur.dl[j] : 0.f;
      float Bv[NS], Cv[NS];
      if (kPipe) {
        bc_row<NS>(bcs[wave], j, Bv, Cv);
      } else {
        const size_t row = (size_t)(tc + min(j, nv - 1)) * sh.ld_bc;
        load_row<NS>(Bb + row, Bv);
        if (need_g) load_row<NS>(Cb + row, Cv);
      }
      const float du = ok ? dlj * cur.uu[j] : 0.f;
      if (need_g) {
        const float dy = ok ? cur.gr[j] * cur.zr[j] * sigmoid(cur.zr[j]) : 0.f;
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          const float a = fast_exp2(dlj * A2[n]);
          h[n] = fmaf(a, h[n], du * Bv[n]);
          P[n] *= a;
          G[n] = fmaf(P[n], dy * Cv[n], G[n]);
        }
      } else {
#pragma unroll
        for (int n = 0; n < NS; ++n) h[n] = fmaf(fast_exp2(dlj * A2[n]), h[n], du * Bv[n]);
      }
      sd += dlj;
    }
    if (kPipe) {
      if (more) {
#pragma unroll
        for (int q = 0; q < kBcPer; ++q) mybc[lane + kWave * q] = bc_next[q];
        wave_sync();
        cur = nxt;
      }
    } else if (more) {
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        cur.dl[j] = nxt.dl[j];
        cur.uu[j] = nxt.uu[j];
      }
    }
  }

  if (!active) return;
  const size_t sg = (size_t)b * sh.nseg + s;
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    seg_h[(sg * NS + n) * Di + d] = h[n];
    if (BWD) seg_g[(sg * NS + n) * Di + d] = G[n];
  }
  seg_sd[sg * Di + d] = sd;
}

// 1'. segment summaries when the states before every chunk are given (the
// forward's checkpoints): the main sweep starts each chunk from them, so a
// segment only needs its delta sum and its adjoint summary
// G = sum_t exp(A S_t) dy_t C_t, S_t the delta sum of the segment's steps up to
// and including t (the running decay product of the summary above, taken as one
// exponential of the running sum).  u and B are not read.  Segment 0's summary
// is never used, so the grid starts at segment 1.
template <typename T, int NS>
__global__ __launch_bounds__(kBlock) void scan_gsum(const T* __restrict__ delta, const float* __restrict__ A_log,
                                                    const T* __restrict__ Cm, const T* __restrict__ z,
                                                    const T* __restrict__ dout, float* __restrict__ seg_g,
                                                    float* __restrict__ seg_sd, ScanShape sh) {
  const int d = blockIdx.x * kBlock + threadIdx.x;
  const int s = blockIdx.y + 1, b = blockIdx.z;
  if (d >= sh.Di) return;
  const int Di = sh.Di;
  float A2[NS], G[NS];
  load_A2<NS>(A_log, d, A2);
#pragma unroll
  for (int n = 0; n < NS; ++n) G[n] = 0.f;
  float S = 0.f;
  const int t0 = s * sh.seg, t1 = min(sh.T, t0 + sh.seg);
  const size_t bo = (size_t)b * sh.T * Di;
  const T* __restrict__ db = delta + bo;
  const T* __restrict__ gb = dout + bo;
  const T* __restrict__ zb = z + (size_t)b * sh.T * sh.ld_z;
  const T* __restrict__ Cb = Cm + (size_t)b * sh.T * sh.ld_bc;
  // bf16: each chunk's delta, d_out and z are loaded one chunk ahead (without
  // it the kernel spent 78 % of its wave time waiting on these loads); float
  // loads them at the chunk's start (its prefetch measured slower).  A ragged
  // last chunk reads its last step again, with zero weight.
  constexpr bool kPre = sizeof(T) == 2;
  float ldl[kChunk], lgr[kChunk], lzz[kChunk];
  const auto load = [&](int tc) {
    const int nv = min(kChunk, t1 - tc);
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const unsigned tj = (unsigned)(tc + min(j, nv - 1));
      ldl[j] = ld(db, tj * Di + d);
      lgr[j] = ld(gb, tj * Di + d);
      lzz[j] = ld(zb, tj * sh.ld_z + d);
    }
  };
  if (kPre) load(t0);
  for (int tc = t0; tc < t1; tc += kChunk) {
    const int nv = min(kChunk, t1 - tc);
    if (!kPre) load(tc);
    float dl[kChunk], dy[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      dl[j] = j < nv ? ldl[j] : 0.f;
      dy[j] = j < nv ? lgr[j] * lzz[j] * sigmoid(lzz[j]) : 0.f;
    }
    if (kPre && tc + kChunk < t1) load(tc + kChunk);
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      float Cv[NS];
      load_row<NS>(Cb + (size_t)(tc + min(j, nv - 1)) * sh.ld_bc, Cv);
      S += dl[j];
#pragma unroll
      for (int n = 0; n < NS; ++n) G[n] = fmaf(fast_exp2(A2[n] * S), dy[j] * Cv[n], G[n]);
    }
  }
  const size_t sg = (size_t)b * sh.nseg + s;
#pragma unroll
  for (int n = 0; n < NS; ++n) seg_g[(sg * NS + n) * Di + d] = G[n];
  seg_sd[sg * Di + d] = S;
}

// ---------------------------------------------------------------------------
// 2. carries across segments, one thread per (b, n, d), in place.  Segment s's
// decay is exp(A * sum of its delta); the forward carry (FWD) runs over s
// ascending, the adjoint carry (BWD) descending.  Each group of segments' loads
// goes out before the group's stores (a load behind a store to the same array
// would otherwise wait for it), so a thread pays one memory round trip per group.
constexpr int kCarryGroup = 8;

template <int NS, bool FWD, bool BWD>
__global__ __launch_bounds__(kBlock) void scan_carry(const float* __restrict__ A_log, float* __restrict__ seg_h,
                                                     float* __restrict__ seg_g, const float* __restrict__ seg_sd,
                                                     ScanShape sh) {
  const int idx = blockIdx.x * kBlock + threadIdx.x;
  const int Di = sh.Di;
  if (idx >= sh.Bt * NS * Di) return;
  const int d = idx % Di, n = (idx / Di) % NS, b = idx / (Di * NS);
  const float A2 = -expf(A_log[(size_t)d * NS + n]) * kLog2e;
  const size_t sd0 = (size_t)b * sh.nseg * Di + d;
  const size_t h0 = ((size_t)b * sh.nseg * NS + n) * Di + d;
  const size_t hs = (size_t)NS * Di;
  float H = 0.f;
  for (int s0 = 0; FWD && s0 < sh.nseg; s0 += kCarryGroup) {
    float sd[kCarryGroup], loc[kCarryGroup];
#pragma unroll
    for (int j = 0; j < kCarryGroup; ++j) {  // past the last segment: repeat it (never used)
      const size_t s = (size_t)min(s0 + j, sh.nseg - 1);
      sd[j] = seg_sd[sd0 + s * Di];
      loc[j] = seg_h[h0 + s * hs];
    }
#pragma unroll
    for (int j = 0; j < kCarryGroup; ++j) {
      if (s0 + j < sh.nseg) {
        seg_h[h0 + (size_t)(s0 + j) * hs] = H;
        H = fmaf(fast_exp2(A2 * sd[j]), H, loc[j]);
      }
    }
  }
  if (!BWD) return;
  // the adjoint leaving segment s; segment 0's own summary is not needed
  float G = 0.f;
  for (int s0 = sh.nseg - 1; s0 >= 1; s0 -= kCarryGroup) {
    float sd[kCarryGroup], loc[kCarryGroup];
#pragma unroll
    for (int j = 0; j < kCarryGroup; ++j) {  // below segment 1: repeat it (never used)
      const size_t s = (size_t)max(s0 - j, 1);
      sd[j] = seg_sd[sd0 + s * Di];
      loc[j] = seg_g[h0 + s * hs];
    }
#pragma unroll
    for (int j = 0; j < kCarryGroup; ++j) {
      if (s0 - j >= 1) {
        seg_g[h0 + (size_t)(s0 - j) * hs] = G;
        G = fmaf(fast_exp2(A2 * sd[j]), G, loc[j]);
      }
    }
  }
  seg_g[h0] = G;
}

// ---------------------------------------------------------------------------
// 3. the backward sweep of one segment.
//
// Per chunk, a_t h_{t-1} of the later kRegSteps steps stays in registers; for
// d_state = 16 the earlier steps' values go to LDS (each lane reads back only
// its own slots, so no barrier is needed), which keeps two blocks per CU.
template <int NS>
struct ChunkTile {
  static constexpr int kRegSteps = (NS * kChunk <= 64) ? kChunk : 64 / NS;
  static constexpr int kLdsSteps = kChunk - kRegSteps;
};

// The float sweep, and the bf16 one when the chunk states are given.  bf16
// rebuilding its own states takes the lane-pair sweep below: measured 9 %
// faster there (1.19 against 1.30 ms on batch 2, 8192 steps, 5120 channels),
// while from given states the lane pairs run 4-6 % slower (1.09 against 1.05
// ms on that shape, 0.67 against 0.63 ms on batch 8, 2048 steps, 3072
// channels) and on float storage 3 % slower.  Two waves per SIMD.
// GCK: `ckpt` holds the exact state before every chunk (the forward's
// checkpoints) instead of the local ones of the summary pass; seg_h, ckpt_sd
// are then unused.
template <typename T, int NS, bool SOFTPLUS, bool GCK>
__global__ __launch_bounds__(kBlock, sizeof(T) == 4 ? 2 : 1) void scan_bwd_main(
    const T* __restrict__ u, const T* __restrict__ delta, const float* __restrict__ A_log,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dp,
    const T* __restrict__ z, const T* __restrict__ dout, T* __restrict__ d_u,
    T* __restrict__ d_delta, T* __restrict__ d_z, const float* __restrict__ ckpt,
    const float* __restrict__ ckpt_sd, const float* __restrict__ seg_h, const float* __restrict__ seg_g,
    float* __restrict__ part_bc, float* __restrict__ part_a, ScanShape sh) {
  static_assert(sizeof(T) == 4 || GCK, "bf16 rebuilding its states takes the lane-pair sweep");
  constexpr int kLogNS = NS == 16 ? 4 : NS == 8 ? 3 : NS == 4 ? 2 : NS == 2 ? 1 : 0;
  constexpr int kRep = kWave / NS;  // lanes holding each reduced value
  constexpr int kReg = ChunkTile<NS>::kRegSteps;
  constexpr int kLds = ChunkTile<NS>::kLdsSteps;
  static_assert(NS % 4 == 0, "a*h rows move through LDS as float4");
  __shared__ float red[2][kBlock / kWave][kChunk][2 * NS];
  __shared__ float4 lds_ah[kLds > 0 ? kLds : 1][NS / 4][kBlock];
  __shared__ __align__(16) float bcs[2][kChunk][2 * NS];
  __shared__ float red_sink[kBlock];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int d = blockIdx.x * kBlock + tid;
  const int s = blockIdx.y, b = blockIdx.z;
  const bool active = d < sh.Di;
  const int dc = active ? d : sh.Di - 1;
  const int Di = sh.Di;
  const size_t row0 = (size_t)b * sh.T;
  const size_t sg = (size_t)b * sh.nseg + s;

  float A2[NS];
  load_A2<NS>(A_log, dc, A2);
  const float Dd = Dp[dc];
  float g[NS], dA[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    g[n] = (s == sh.nseg - 1) ? 0.f : seg_g[(sg * NS + n) * Di + dc];
    dA[n] = 0.f;
  }
  float dD = 0.f;

  const int t0 = s * sh.seg, t1 = min(sh.T, t0 + sh.seg);
  const int c_first = t0 / kChunk, c_last = (t1 - 1) / kChunk;
  const T* __restrict__ Bb = Bm + row0 * sh.ld_bc;
  const T* __restrict__ Cb = Cm + row0 * sh.ld_bc;
  // the last chunk's B | C rows go to LDS before the sweep, and each chunk
  // fetches the next one's while it computes
  if (tid < kChunk * 2 * NS)
    (&bcs[c_last & 1][0][0])[tid] =
        bc_element<T, NS>(Bb, Cb, sh.ld_bc, c_last * kChunk, min(kChunk, t1 - c_last * kChunk), tid);
  __syncthreads();
  // a chunk's loads: its per-step channel values (delta, u, z, d_out) and, when
  // the states are given, its starting state.  With given states the next
  // chunk's loads go out at the end of the current one, before its barrier, into
  // registers it no longer needs (measured: 2-3 % off the sweep); a sweep that
  // rebuilds its states issues them at the chunk's start (earlier costs bf16 a
  // tenth and float nothing).
  // Per-step rows addressed as scalar row pointer + 32-bit lane offset with
  // given states (measured in the ISA: 4 % fewer VALU instructions); the sweep
  // that rebuilds its states keeps 64-bit lane addresses, which spill less there.
  constexpr bool kRowAddr = GCK;
  float dl[kChunk], uu[kChunk], zr[kChunk], gr[kChunk], dy[kChunk];
  float hg[NS];
  const auto load_chunk = [&](int c) {
    const int tc = c * kChunk;
    const int nv = min(kChunk, t1 - tc);
    if (GCK) {
      const size_t cc = (size_t)b * sh.nchunk + c;
#pragma unroll
      for (int n = 0; n < NS; ++n) hg[n] = ckpt[(cc * NS + n) * Di + dc];
    }
    // steps past a ragged chunk's end read its last step again (unused)
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const size_t tj = row0 + tc + min(j, nv - 1);
      if (kRowAddr) {
        const size_t r = tj * Di;
        dl[j] = ld_row(delta + r, dc);
        uu[j] = ld_row(u + r, dc);
        zr[j] = ld_row(z + tj * sh.ld_z, dc);
        gr[j] = ld_row(dout + r, dc);
      } else {
        const size_t i = tj * Di + dc;
        dl[j] = ld(delta, i);
        uu[j] = ld(u, i);
        zr[j] = ld(z, tj * sh.ld_z + dc);
        gr[j] = ld(dout, i);
      }
    }
  };
  if (GCK) load_chunk(c_last);
  for (int c = c_last; c >= c_first; --c) {
    const int tc = c * kChunk;
    const int nv = min(kChunk, t1 - tc);
    const int buf = c & 1;
    const float bc_next = c > c_first ? bc_element<T, NS>(Bb, Cb, sh.ld_bc, tc - kChunk, kChunk, tid) : 0.f;
    // state before the chunk: given, or local checkpoint + decayed carry-in
    float h[NS];
    if (GCK) {
#pragma unroll
      for (int n = 0; n < NS; ++n) h[n] = hg[n];
    } else if (c == c_first) {
#pragma unroll
      for (int n = 0; n < NS; ++n) h[n] = (s == 0) ? 0.f : seg_h[(sg * NS + n) * Di + dc];
    } else {
      const size_t cc = (size_t)b * sh.nchunk + c;
      const float sdv = ckpt_sd[cc * Di + dc];
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        const float hin = (s == 0) ? 0.f : seg_h[(sg * NS + n) * Di + dc];
        h[n] = fmaf(fast_exp2(A2[n] * sdv), hin, ckpt[(cc * NS + n) * Di + dc]);
      }
    }
    // the gate math (dy = d_out SiLU(z) and the d_z factor) waits for the loads
    // step by step
    if (!GCK) load_chunk(c);
    // forward: rebuild the chunk's states, keep a_t h_{t-1}
    float ah[kReg][NS];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      if (j < nv) {
        float Bv[NS], Cv[NS];
        bc_row<NS>(bcs[buf], j, Bv, Cv);
        const float sz = sigmoid(zr[j]);
        dy[j] = active ? gr[j] * zr[j] * sz : 0.f;
        const float dzf = gr[j] * sz * (1.f + zr[j] * (1.f - sz));
        const float du = dl[j] * uu[j];
        float y = Dd * uu[j];
        float dC[NS];
        float aj[NS];
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          const float a = fast_exp2(dl[j] * A2[n]);
          aj[n] = a * h[n];
          h[n] = fmaf(du, Bv[n], aj[n]);
          y = fmaf(Cv[n], h[n], y);
          dC[n] = dy[j] * h[n];
        }
        if (j < kLds) {
#pragma unroll
          for (int q = 0; q < NS / 4; ++q)
            lds_ah[j < kLds ? j : 0][q][tid] = make_float4(aj[4 * q], aj[4 * q + 1], aj[4 * q + 2], aj[4 * q + 3]);
        } else {
#pragma unroll
          for (int n = 0; n < NS; ++n) ah[j >= kLds ? j - kLds : 0][n] = aj[n];
        }
        if (active) {
          if (kRowAddr) st_row(d_z + (row0 + tc + j) * sh.ld_z, d, y * dzf);
          else st(d_z, (row0 + tc + j) * sh.ld_z + d, y * dzf);
        }
        wave_reduce_scatter<NS>(dC, lane);
        // one lane of each group of kRep holds the sum; the others write to
        // their own sink slot (an address select instead of a lane branch)
        *((lane & (kRep - 1)) == 0 ? &red[buf][wave][j][NS + (lane >> (6 - kLogNS))] : &red_sink[tid]) = dC[0];
      }
    }
    // The reverse walk reads B | C again rather than keeping the forward's
    // values: without this compiler barrier they would be reused, live across
    // the walks (8 steps x 2N registers).
    asm volatile("" ::: "memory");
    // reverse: adjoint through the chunk
#pragma unroll
    for (int j = kChunk - 1; j >= 0; --j) {
      if (j < nv) {
        float Bv[NS], Cv[NS];
        bc_row<NS>(bcs[buf], j, Bv, Cv);
        float aj[NS];
        if (j < kLds) {
#pragma unroll
          for (int q = 0; q < NS / 4; ++q) {
            const float4 v = lds_ah[j < kLds ? j : 0][q][tid];
            aj[4 * q] = v.x;
            aj[4 * q + 1] = v.y;
            aj[4 * q + 2] = v.z;
            aj[4 * q + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int n = 0; n < NS; ++n) aj[n] = ah[j >= kLds ? j - kLds : 0][n];
        }
        // delta of the step, opaque to the compiler: a_t is recomputed here
        // rather than kept from the forward walk (8 steps x N live registers)
        float dlr = dl[j];
        asm volatile("" : "+v"(dlr));
        const float du = active ? dlr * uu[j] : 0.f;
        float sgb = 0.f, saw = 0.f;
        float dB[NS];
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          const float gn = fmaf(dy[j], Cv[n], g[n]);
          const float w = gn * aj[n];
          saw = fmaf(A2[n], w, saw);
          dA[n] = fmaf(dl[j], w, dA[n]);
          sgb = fmaf(gn, Bv[n], sgb);
          dB[n] = gn * du;
          g[n] = fast_exp2(dlr * A2[n]) * gn;
        }
        float ddl = fmaf(saw, kLn2, uu[j] * sgb);
        if (SOFTPLUS) ddl = dl[j] > 20.f ? ddl : ddl * (1.f - fast_exp2(-dl[j] * kLog2e));
        dD = fmaf(dy[j], uu[j], dD);
        if (active) {
          const size_t r = (row0 + tc + j) * Di;
          if (kRowAddr) {
            st_row(d_u + r, d, fmaf(Dd, dy[j], dl[j] * sgb));
            st_row(d_delta + r, d, ddl);
          } else {
            st(d_u, r + d, fmaf(Dd, dy[j], dl[j] * sgb));
            st(d_delta, r + d, ddl);
          }
        }
        wave_reduce_scatter<NS>(dB, lane);
        *((lane & (kRep - 1)) == 0 ? &red[buf][wave][j][lane >> (6 - kLogNS)] : &red_sink[tid]) = dB[0];
      }
    }
    if (GCK && c > c_first) load_chunk(c - 1);
    // the buffer written here was last read before the previous chunk's barrier
    if (c > c_first && tid < kChunk * 2 * NS) (&bcs[buf ^ 1][0][0])[tid] = bc_next;
    __syncthreads();
    for (int q = tid; q < kChunk * 2 * NS; q += kBlock) {
      const int j = q / (2 * NS), k = q - j * (2 * NS);
      if (j < nv) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < kBlock / kWave; ++w) acc += red[buf][w][j][k];
        part_bc[(((size_t)blockIdx.x * sh.Bt + b) * sh.T + tc + j) * 2 * NS + k] = acc;
      }
    }
  }
  if (!active) return;
#pragma unroll
  for (int n = 0; n < NS; ++n) part_a[(sg * (NS + 1) + n) * Di + d] = dA[n];
  part_a[(sg * (NS + 1) + NS) * Di + d] = dD;
}


// 3'. the main sweep on lane pairs (bf16 storage).  Lanes 2i and 2i+1 of a wave share the
// channels d = 2i and 2i+1: lane l owns channel l (its per-step loads, gate
// math and outputs) and holds, for both channels, the half of the states with
// index in [NH q, NH q + NH), q = l & 1.  The d_B | d_C sums over channels then
// cross only the 32 lanes of one state half (half the values per lane of the
// one-channel-per-lane layout, so half the cross-lane work), and each
// per-channel sum over states (y, sum g B, sum A a h g) takes one DPP add
// across the pair.  The partner channel's delta, delta u and dy come over by
// DPP.  Register roles: index 0 holds the lane's own channel, index 1 the
// partner's, so the partner's partial for this lane's channel is always its
// index-1 value.
template <int NS>
__device__ __forceinline__ void bc_half(const float (&bcs)[kChunk][2 * NS], int j, int n0, float (&Bv)[NS / 2],
                                        float (&Cv)[NS / 2]) {
  constexpr int NH = NS / 2;
  if constexpr (NH % 4 == 0) {
    const float4* pb = reinterpret_cast<const float4*>(&bcs[j][n0]);
    const float4* pc = reinterpret_cast<const float4*>(&bcs[j][NS + n0]);
#pragma unroll
    for (int k = 0; k < NH / 4; ++k) {
      const float4 b = pb[k], c = pc[k];
      Bv[4 * k] = b.x; Bv[4 * k + 1] = b.y; Bv[4 * k + 2] = b.z; Bv[4 * k + 3] = b.w;
      Cv[4 * k] = c.x; Cv[4 * k + 1] = c.y; Cv[4 * k + 2] = c.z; Cv[4 * k + 3] = c.w;
    }
  } else {
    const float2* pb = reinterpret_cast<const float2*>(&bcs[j][n0]);
    const float2* pc = reinterpret_cast<const float2*>(&bcs[j][NS + n0]);
#pragma unroll
    for (int k = 0; k < NH / 2; ++k) {
      const float2 b = pb[k], c = pc[k];
      Bv[2 * k] = b.x; Bv[2 * k + 1] = b.y;
      Cv[2 * k] = c.x; Cv[2 * k + 1] = c.y;
    }
  }
}

template <typename T, int NS, bool SOFTPLUS>
__global__ __launch_bounds__(kBlock, 2) void scan_bwd_pair(
    const T* __restrict__ u, const T* __restrict__ delta, const float* __restrict__ A_log,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dp,
    const T* __restrict__ z, const T* __restrict__ dout, T* __restrict__ d_u,
    T* __restrict__ d_delta, T* __restrict__ d_z, const float* __restrict__ ckpt,
    const float* __restrict__ ckpt_sd, const float* __restrict__ seg_h, const float* __restrict__ seg_g,
    float* __restrict__ part_bc, float* __restrict__ part_a, ScanShape sh) {
  static_assert(sizeof(T) == 2, "the lane-pair sweep is the bf16 path");
  constexpr int NH = NS / 2;
  // with d_state 16 one more step of a_t h_{t-1} stays in registers than in the
  // one-channel sweep (the half-row B | C leave room: 249 VGPRs, no spills;
  // measured 0.5-0.8 % faster)
  constexpr int kReg = ChunkTile<NS>::kRegSteps + (NS == 16 ? 1 : 0);
  constexpr int kLds = kChunk - kReg;
  static_assert(NS % 4 == 0, "a*h rows move through LDS as float4");
  __shared__ float red[2][kBlock / kWave][kChunk][2 * NS];
  __shared__ float4 lds_ah[kLds > 0 ? kLds : 1][NS / 4][kBlock];
  __shared__ __align__(16) float bcs[2][kChunk][2 * NS];
  __shared__ float red_sink[kBlock];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int n0 = (lane & 1) * NH;  // first state of this lane's half
  const int d = blockIdx.x * kBlock + tid, dq = d ^ 1;
  const int s = blockIdx.y, b = blockIdx.z;
  const int Di = sh.Di;
  const bool active = d < Di, active_q = dq < Di;
  const int dc = active ? d : Di - 1, dqc = active_q ? dq : Di - 1;
  const size_t row0 = (size_t)b * sh.T;
  const size_t sg = (size_t)b * sh.nseg + s;
  const bool last_seg = s == sh.nseg - 1;
  // [.., N, Di] state blocks: element (n0 + k, channel) at lane element offset
  // o0 | o1 and wave-uniform byte offset k Di 4 from the block
  const uint32_t o0 = (uint32_t)(n0 * Di + dc), o1 = (uint32_t)(n0 * Di + dqc);
  const uint32_t row_bytes = (uint32_t)Di * 4u;
  const BufRes rsh = buf_res(seg_h + sg * NS * Di);

  float A2[2][NH];
#pragma unroll
  for (int k = 0; k < NH; ++k) {
    A2[0][k] = -expf(A_log[(size_t)dc * NS + n0 + k]) * kLog2e;
    A2[1][k] = -expf(A_log[(size_t)dqc * NS + n0 + k]) * kLog2e;
  }
  const float Dd = Dp[dc];
  float g[2][NH], dA[2][NH];
  const BufRes rsg = buf_res(seg_g + sg * NS * Di);
#pragma unroll
  for (int k = 0; k < NH; ++k) {
    g[0][k] = last_seg ? 0.f : buf_ld<float>(rsg, o0, k * row_bytes);
    g[1][k] = last_seg ? 0.f : buf_ld<float>(rsg, o1, k * row_bytes);
    dA[0][k] = 0.f;
    dA[1][k] = 0.f;
  }
  float dD = 0.f;

  const int t0 = s * sh.seg, t1 = min(sh.T, t0 + sh.seg);
  const int c_first = t0 / kChunk, c_last = (t1 - 1) / kChunk;
  const T* __restrict__ Bb = Bm + row0 * sh.ld_bc;
  const T* __restrict__ Cb = Cm + row0 * sh.ld_bc;
  // the last chunk's B | C rows go to LDS before the sweep; each chunk fetches
  // the next one's while it computes
  if (tid < kChunk * 2 * NS)
    (&bcs[c_last & 1][0][0])[tid] =
        bc_element<T, NS>(Bb, Cb, sh.ld_bc, c_last * kChunk, min(kChunk, t1 - c_last * kChunk), tid);
  __syncthreads();
  // a chunk's loads: its per-step values of the lane's own channel (delta, u,
  // z, d_out), issued at the chunk's start.  Rows of a chunk sit at
  // wave-uniform byte offsets from the chunk's first row.
  const uint32_t step_bytes = (uint32_t)(Di * sizeof(T)), zstep_bytes = (uint32_t)(sh.ld_z * sizeof(T));
  float dl[kChunk], uu[kChunk], zr[kChunk], gr[kChunk], dy[kChunk];
  const auto load_chunk = [&](int c) {
    const int tc = c * kChunk;
    const int nv = min(kChunk, t1 - tc);
    const size_t rowc = row0 + tc;
    const BufRes rd = buf_res(delta + rowc * Di), ru = buf_res(u + rowc * Di), rg = buf_res(dout + rowc * Di);
    const BufRes rz = buf_res(z + rowc * sh.ld_z);
    // steps past a ragged chunk's end read its last step again (unused)
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const uint32_t jj = (uint32_t)min(j, nv - 1);
      dl[j] = buf_ld<T>(rd, dc, jj * step_bytes);
      uu[j] = buf_ld<T>(ru, dc, jj * step_bytes);
      zr[j] = buf_ld<T>(rz, dc, jj * zstep_bytes);
      gr[j] = buf_ld<T>(rg, dc, jj * step_bytes);
    }
  };
  for (int c = c_last; c >= c_first; --c) {
    const int tc = c * kChunk;
    const int nv = min(kChunk, t1 - tc);
    const int buf = c & 1;
    const float bc_next = c > c_first ? bc_element<T, NS>(Bb, Cb, sh.ld_bc, tc - kChunk, kChunk, tid) : 0.f;
    // states before the chunk: local checkpoint + decayed carry-in
    float h[2][NH];
    if (c == c_first) {
#pragma unroll
      for (int k = 0; k < NH; ++k) {
        h[0][k] = (s == 0) ? 0.f : buf_ld<float>(rsh, o0, k * row_bytes);
        h[1][k] = (s == 0) ? 0.f : buf_ld<float>(rsh, o1, k * row_bytes);
      }
    } else {
      // local checkpoint + carry-in decayed over the segment's steps before the chunk
      const size_t cc = (size_t)b * sh.nchunk + c;
      const BufRes rsd = buf_res(ckpt_sd + cc * Di), rc = buf_res(ckpt + cc * NS * Di);
      const float sd0 = buf_ld<float>(rsd, dc, 0), sd1 = buf_ld<float>(rsd, dqc, 0);
#pragma unroll
      for (int k = 0; k < NH; ++k) {
        const float hin0 = (s == 0) ? 0.f : buf_ld<float>(rsh, o0, k * row_bytes);
        const float hin1 = (s == 0) ? 0.f : buf_ld<float>(rsh, o1, k * row_bytes);
        h[0][k] = fmaf(fast_exp2(A2[0][k] * sd0), hin0, buf_ld<float>(rc, o0, k * row_bytes));
        h[1][k] = fmaf(fast_exp2(A2[1][k] * sd1), hin1, buf_ld<float>(rc, o1, k * row_bytes));
      }
    }
    load_chunk(c);
    const BufRes rdz = buf_res(d_z + (row0 + tc) * sh.ld_z);
    const BufRes rdu = buf_res(d_u + (row0 + tc) * Di), rdd = buf_res(d_delta + (row0 + tc) * Di);
    // forward: rebuild the chunk's states, keep a_t h_{t-1}
    float ah[kReg][NS];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      if (j < nv) {
        float Bv[NH], Cv[NH];
        bc_half<NS>(bcs[buf], j, n0, Bv, Cv);
        const float sz = sigmoid(zr[j]);
        dy[j] = active ? gr[j] * zr[j] * sz : 0.f;
        const float dzf = gr[j] * sz * (1.f + zr[j] * (1.f - sz));
        const float du = dl[j] * uu[j];
        const float dlq = dpp<kQuadXor1>(dl[j]), duq = dpp<kQuadXor1>(du), dyq = dpp<kQuadXor1>(dy[j]);
        float y0, y1;
        float dC[NH], aj[NS];
#pragma unroll
        for (int k = 0; k < NH; ++k) {
          aj[k] = fast_exp2(dl[j] * A2[0][k]) * h[0][k];
          h[0][k] = fmaf(du, Bv[k], aj[k]);
          y0 = k == 0 ? Cv[k] * h[0][k] : fmaf(Cv[k], h[0][k], y0);
          aj[NH + k] = fast_exp2(dlq * A2[1][k]) * h[1][k];
          h[1][k] = fmaf(duq, Bv[k], aj[NH + k]);
          y1 = k == 0 ? Cv[k] * h[1][k] : fmaf(Cv[k], h[1][k], y1);
          dC[k] = fmaf(dyq, h[1][k], dy[j] * h[0][k]);
        }
        // this lane's channel: its own half of the states plus the partner's
        // partial over the other half
        const float y = fmaf(Dd, uu[j], y0 + dpp<kQuadXor1>(y1));
        if (j < kLds) {
#pragma unroll
          for (int v = 0; v < NS / 4; ++v)
            lds_ah[j < kLds ? j : 0][v][tid] = make_float4(aj[4 * v], aj[4 * v + 1], aj[4 * v + 2], aj[4 * v + 3]);
        } else {
#pragma unroll
          for (int k = 0; k < NS; ++k) ah[j >= kLds ? j - kLds : 0][k] = aj[k];
        }
        if (active) buf_st<T>(rdz, d, j * zstep_bytes, y * dzf);
        pair_reduce_scatter<NH>(dC, lane);
        *(pair_writer<NH>(lane) ? &red[buf][wave][j][NS + n0 + pair_index<NH>(lane)] : &red_sink[tid]) = dC[0];
      }
    }
    // The reverse walk reads B | C again rather than keeping the forward's
    // values live across the walks.
    asm volatile("" ::: "memory");
    // reverse: adjoint through the chunk
#pragma unroll
    for (int j = kChunk - 1; j >= 0; --j) {
      if (j < nv) {
        float Bv[NH], Cv[NH];
        bc_half<NS>(bcs[buf], j, n0, Bv, Cv);
        float aj[NS];
        if (j < kLds) {
#pragma unroll
          for (int v = 0; v < NS / 4; ++v) {
            const float4 w4 = lds_ah[j < kLds ? j : 0][v][tid];
            aj[4 * v] = w4.x;
            aj[4 * v + 1] = w4.y;
            aj[4 * v + 2] = w4.z;
            aj[4 * v + 3] = w4.w;
          }
        } else {
#pragma unroll
          for (int k = 0; k < NS; ++k) aj[k] = ah[j >= kLds ? j - kLds : 0][k];
        }
        // deltas of the step, opaque to the compiler: a_t is recomputed here
        // rather than kept from the forward walk
        float dlr = dl[j], dlqr = dpp<kQuadXor1>(dl[j]);
        asm volatile("" : "+v"(dlr), "+v"(dlqr));
        const float du = active ? dlr * uu[j] : 0.f;
        const float duq = dpp<kQuadXor1>(du), dyq = dpp<kQuadXor1>(dy[j]);
        float sgb0, sgb1, saw0, saw1;
        float dB[NH];
#pragma unroll
        for (int k = 0; k < NH; ++k) {
          const float gn0 = fmaf(dy[j], Cv[k], g[0][k]);
          const float w0 = gn0 * aj[k];
          saw0 = k == 0 ? A2[0][k] * w0 : fmaf(A2[0][k], w0, saw0);
          dA[0][k] = fmaf(dlr, w0, dA[0][k]);
          sgb0 = k == 0 ? gn0 * Bv[k] : fmaf(gn0, Bv[k], sgb0);
          g[0][k] = fast_exp2(dlr * A2[0][k]) * gn0;
          const float gn1 = fmaf(dyq, Cv[k], g[1][k]);
          const float w1 = gn1 * aj[NH + k];
          saw1 = k == 0 ? A2[1][k] * w1 : fmaf(A2[1][k], w1, saw1);
          dA[1][k] = fmaf(dlqr, w1, dA[1][k]);
          sgb1 = k == 0 ? gn1 * Bv[k] : fmaf(gn1, Bv[k], sgb1);
          g[1][k] = fast_exp2(dlqr * A2[1][k]) * gn1;
          dB[k] = fmaf(gn1, duq, gn0 * du);
        }
        const float sgb = sgb0 + dpp<kQuadXor1>(sgb1);
        const float saw = saw0 + dpp<kQuadXor1>(saw1);
        float ddl = fmaf(saw, kLn2, uu[j] * sgb);
        if (SOFTPLUS) ddl = dl[j] > 20.f ? ddl : ddl * (1.f - fast_exp2(-dl[j] * kLog2e));
        dD = fmaf(dy[j], uu[j], dD);
        if (active) {
          buf_st<T>(rdu, d, j * step_bytes, fmaf(Dd, dy[j], dl[j] * sgb));
          buf_st<T>(rdd, d, j * step_bytes, ddl);
        }
        pair_reduce_scatter<NH>(dB, lane);
        *(pair_writer<NH>(lane) ? &red[buf][wave][j][n0 + pair_index<NH>(lane)] : &red_sink[tid]) = dB[0];
      }
    }
    // the buffer written here was last read before the previous chunk's barrier
    if (c > c_first && tid < kChunk * 2 * NS) (&bcs[buf ^ 1][0][0])[tid] = bc_next;
    __syncthreads();
    for (int v = tid; v < kChunk * 2 * NS; v += kBlock) {
      const int j = v / (2 * NS), k = v - j * (2 * NS);
      if (j < nv) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < kBlock / kWave; ++w) acc += red[buf][w][j][k];
        part_bc[(((size_t)blockIdx.x * sh.Bt + b) * sh.T + tc + j) * 2 * NS + k] = acc;
      }
    }
  }
  // each (channel, state) of the lane pair is written by exactly one lane
  const BufRes rpa = buf_res(part_a + sg * (NS + 1) * Di);
#pragma unroll
  for (int k = 0; k < NH; ++k) {
    if (active) buf_st<float>(rpa, o0, k * row_bytes, dA[0][k]);
    if (active_q) buf_st<float>(rpa, o1, k * row_bytes, dA[1][k]);
  }
  if (active) buf_st<float>(rpa, d, NS * row_bytes, dD);
}

// ---------------------------------------------------------------------------
// 4. fixed-order sums of the partials.  Blocks [0, nblk_bc) sum the d_B | d_C
// block partials over channel tiles; the rest sum the d_A_log | d_D segment
// partials of 64 channels of one state, four thread groups taking every fourth
// partial, combined in LDS in group order.
template <typename T, int NS>
__global__ __launch_bounds__(kBlock) void scan_bwd_finalize(
    const float* __restrict__ A_log, T* __restrict__ d_B, T* __restrict__ d_C,
    float* __restrict__ d_A_log, float* __restrict__ d_D, const float* __restrict__ part_bc,
    const float* __restrict__ part_a, ScanShape sh, int nblk_bc, int accumulate) {
  __shared__ float grp_sum[kBlock / kWave][kWave];
  if ((int)blockIdx.x < nblk_bc) {
    const size_t rows = (size_t)sh.Bt * sh.T;
    const size_t idx = (size_t)blockIdx.x * kBlock + threadIdx.x;
    if (idx >= rows * 2 * NS) return;
    const size_t r = idx / (2 * NS);
    const int k = (int)(idx - r * 2 * NS);
    float acc = 0.f;
#pragma unroll 8
    for (int tile = 0; tile < sh.ntile; ++tile) acc += part_bc[((size_t)tile * rows + r) * 2 * NS + k];
    if (k < NS) st(d_B, r * sh.ld_dbc + k, acc);
    else st(d_C, r * sh.ld_dbc + (k - NS), acc);
  } else {
    const int ndt = (sh.Di + kWave - 1) / kWave;
    const int blk = blockIdx.x - nblk_bc;
    const int n = blk / ndt;
    const int lane = threadIdx.x & (kWave - 1), grp = threadIdx.x / kWave;
    const int d = (blk - n * ndt) * kWave + lane;
    float acc = 0.f;
    if (d < sh.Di) {
      const int parts = sh.Bt * sh.nseg;
#pragma unroll 8
      for (int p = grp; p < parts; p += kBlock / kWave) acc += part_a[((size_t)p * (NS + 1) + n) * sh.Di + d];
    }
    grp_sum[grp][lane] = acc;
    __syncthreads();
    if (grp == 0 && d < sh.Di) {
      float tot = 0.f;
#pragma unroll
      for (int g = 0; g < kBlock / kWave; ++g) tot += grp_sum[g][lane];
      float* dst = n < NS ? &d_A_log[(size_t)d * NS + n] : &d_D[d];
      const float v = n < NS ? -expf(A_log[(size_t)d * NS + n]) * tot : tot;
      *dst = accumulate ? *dst + v : v;
    }
  }
}

// ---------------------------------------------------------------------------
// forward with true states: y, out = y*SiLU(z), optional checkpoints.
template <typename T, int NS>
__global__ __launch_bounds__(kBlock) void scan_fwd_main(
    const T* __restrict__ u, const T* __restrict__ delta, const float* __restrict__ A_log,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dp,
    const T* __restrict__ z, T* __restrict__ y, T* __restrict__ out, float* __restrict__ h_ckpt,
    int ckpt_every, int nckpt, const float* __restrict__ seg_h, ScanShape sh) {
  const int d = blockIdx.x * kBlock + threadIdx.x;
  const int s = blockIdx.y, b = blockIdx.z;
  if (d >= sh.Di) return;
  const int Di = sh.Di;
  float A2[NS];
  load_A2<NS>(A_log, d, A2);
  const float Dd = Dp[d];
  const size_t row0 = (size_t)b * sh.T;
  const size_t sg = (size_t)b * sh.nseg + s;
  float h[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) h[n] = (s == 0) ? 0.f : seg_h[(sg * NS + n) * Di + d];
  const int t0 = s * sh.seg, t1 = min(sh.T, t0 + sh.seg);
  if constexpr (sizeof(T) == 2) {
    // bf16: one step at a time (the chunked, prefetching loop below measured
    // 11 % slower here, while it takes float 15 % less time)
    for (int t = t0; t < t1; ++t) {
      if (h_ckpt && t % ckpt_every == 0) {
        const size_t k = (size_t)b * nckpt + t / ckpt_every;
#pragma unroll
        for (int n = 0; n < NS; ++n) h_ckpt[(k * NS + n) * Di + d] = h[n];
      }
      const size_t i = (row0 + t) * Di + d;
      const float dl = ld(delta, i), uu = ld(u, i);
      float Bv[NS], Cv[NS];
      load_row<NS>(Bm + (row0 + t) * sh.ld_bc, Bv);
      load_row<NS>(Cm + (row0 + t) * sh.ld_bc, Cv);
      const float du = dl * uu;
      float yy = Dd * uu;
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        h[n] = fmaf(fast_exp2(dl * A2[n]), h[n], du * Bv[n]);
        yy = fmaf(Cv[n], h[n], yy);
      }
      if (y) st(y, i, yy);
      if (out) {
        const float zz = ld(z, (row0 + t) * sh.ld_z + d);
        st(out, i, yy * zz * sigmoid(zz));
      }
    }
    return;
  }
  // float: steps go in chunks of kChunk whose delta, u (and z) are loaded one
  // chunk ahead; a ragged last chunk reads its last step again for the unused
  // slots.
  float ndl[kChunk], nuu[kChunk], nzz[kChunk];
  const auto load = [&](int tc) {
    const int nv = min(kChunk, t1 - tc);
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const size_t tj = row0 + tc + min(j, nv - 1);
      ndl[j] = ld(delta, tj * Di + d);
      nuu[j] = ld(u, tj * Di + d);
      if (out) nzz[j] = ld(z, tj * sh.ld_z + d);
    }
  };
  if (t0 < t1) load(t0);
  for (int tc = t0; tc < t1; tc += kChunk) {
    const int nv = min(kChunk, t1 - tc);
    float dl[kChunk], uu[kChunk], zz[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      dl[j] = ndl[j];
      uu[j] = nuu[j];
      zz[j] = out ? nzz[j] : 0.f;
    }
    if (tc + kChunk < t1) load(tc + kChunk);
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      if (j < nv) {
        const int t = tc + j;
        if (h_ckpt && t % ckpt_every == 0) {
          const size_t k = (size_t)b * nckpt + t / ckpt_every;
#pragma unroll
          for (int n = 0; n < NS; ++n) h_ckpt[(k * NS + n) * Di + d] = h[n];
        }
        const size_t i = (row0 + t) * Di + d;
        float Bv[NS], Cv[NS];
        load_row<NS>(Bm + (row0 + t) * sh.ld_bc, Bv);
        load_row<NS>(Cm + (row0 + t) * sh.ld_bc, Cv);
        const float du = dl[j] * uu[j];
        float yy = Dd * uu[j];
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          h[n] = fmaf(fast_exp2(dl[j] * A2[n]), h[n], du * Bv[n]);
          yy = fmaf(Cv[n], h[n], yy);
        }
        if (y) st(y, i, yy);
        if (out) st(out, i, yy * zz[j] * sigmoid(zz[j]));
      }
    }
  }
}

__global__ void fill_zero(float* __restrict__ p, int n) {
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// ---------------------------------------------------------------------------
// host side
namespace {

struct Plan {
  ScanShape sh;
  size_t off[7];
  size_t bytes;
};

// Segment length: the segments of all batch elements and channel tiles run as
// independent blocks of the summary and the main kernel, so a pass takes about
// (rounds of resident blocks) x (segment length + a fixed set-up cost) in each,
// the main kernel's steps weighing about three summary steps (six of the
// adjoint-only summary used when the chunk states are given).  Picks the length,
// a multiple of 8 and at least 64 steps (or the whole sequence), that minimises
// the sum; ties go to the longer segment (fewer carries, less workspace).
int auto_seg(const ssm_dims& dm, long cap_summary, long cap_main, long main_weight) {
  constexpr int kSegOverhead = 16;  // steps' worth of checkpoint restore and carry work
  const long rows = (long)((dm.d_inner + kBlock - 1) / kBlock) * dm.batch;
  const int tmax = (dm.seqlen + kChunk - 1) / kChunk * kChunk;
  const int smin = tmax < 64 ? tmax : 64;
  long best_cost = -1;
  int best = tmax;
  for (int seg = tmax; seg >= smin && seg > 0; seg -= kChunk) {
    const long blocks = rows * ((dm.seqlen + seg - 1) / seg);
    const long rounds = (blocks + cap_summary - 1) / cap_summary + main_weight * ((blocks + cap_main - 1) / cap_main);
    const long cost = rounds * (seg + kSegOverhead);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = seg;
    }
  }
  return best;
}

// CUs of the current device (256 if it cannot be queried)
long device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  return cus;
}

// 256-lane blocks one CU holds at once, from the kernels' register use: the main
// sweep runs two waves per SIMD, the summary two in float and three in bf16
// (its float variant holds the next chunk's values in registers)
long summary_blocks_per_cu(int dtype) { return dtype == SSM_F32 ? 2 : 3; }
constexpr long kMainBlocksPerCU = 2;
// The adjoint-only summary holds seven waves per SIMD in float and five in bf16
// (its prefetch registers); the model keeps seven for both, which picks the
// measured best segment length for batch 2, 8192 steps, 5120 channels (216
// steps; five picks 328, where the main sweep runs 3 % slower).
constexpr long kGsumBlocksPerCU = 7;

int check_dims(const ssm_dims* dm, int dtype) {
  if (!dm) return fail(SSM_ERR_INVALID_ARG, "dims is null");
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (dm->batch < 0 || dm->seqlen < 0 || dm->d_inner <= 0 || dm->d_state <= 0)
    return fail(SSM_ERR_INVALID_ARG, "bad size (batch %d seqlen %d d_inner %d d_state %d)", dm->batch,
                dm->seqlen, dm->d_inner, dm->d_state);
  if (dm->d_state != 4 && dm->d_state != 8 && dm->d_state != 16)
    return fail(SSM_ERR_UNSUPPORTED, "d_state %d not in {4, 8, 16}", dm->d_state);
  if (dm->ld_bc < dm->d_state || dm->ld_dbc < dm->d_state)
    return fail(SSM_ERR_INVALID_ARG, "row strides ld_bc %d / ld_dbc %d below d_state %d", dm->ld_bc, dm->ld_dbc,
                dm->d_state);
  if (dm->ld_z != 0 && dm->ld_z < dm->d_inner)
    return fail(SSM_ERR_INVALID_ARG, "row stride ld_z %d below d_inner %d", dm->ld_z, dm->d_inner);
  // per-sequence offsets are 32-bit in the summary pass
  if ((double)dm->seqlen * (dm->ld_z > dm->d_inner ? dm->ld_z : dm->d_inner) >= 4294967296.0)
    return fail(SSM_ERR_UNSUPPORTED, "seqlen x row stride above 2^32 elements");
  if (dm->seg_len < 0 || dm->seg_len % kChunk != 0)
    return fail(SSM_ERR_INVALID_ARG, "seg_len %d is not 0 or a multiple of %d", dm->seg_len, kChunk);
  if (dtype == SSM_BF16 && ((dm->ld_bc & 1) || (dm->ld_dbc & 1)))
    return fail(SSM_ERR_UNSUPPORTED, "bf16 B/C rows need even strides (ld_bc %d, ld_dbc %d)", dm->ld_bc,
                dm->ld_dbc);
  const double elems = (double)dm->batch * dm->seqlen * (double)(dm->d_inner > dm->ld_bc ? dm->d_inner : dm->ld_bc);
  if (elems > 9.0e15) return fail(SSM_ERR_INVALID_ARG, "tensor too large");
  return SSM_OK;
}

// given_ckpt: the backward takes the chunk states from the caller, so the local
// checkpoints and the forward carry need no workspace.
Plan make_plan(const ssm_dims& dm, int dtype, bool bwd, bool given_ckpt = false) {
  Plan p{};
  ScanShape& sh = p.sh;
  sh.Bt = dm.batch;
  sh.T = dm.seqlen;
  sh.Di = dm.d_inner;
  sh.ld_bc = dm.ld_bc;
  sh.ld_dbc = dm.ld_dbc;
  sh.ld_z = dm.ld_z ? dm.ld_z : dm.d_inner;
  const long cus = dm.seg_len ? 0 : device_cus();
  sh.seg = dm.seg_len ? dm.seg_len
                      : given_ckpt ? auto_seg(dm, cus * kGsumBlocksPerCU, cus * kMainBlocksPerCU, 6)
                                   : auto_seg(dm, cus * summary_blocks_per_cu(dtype), cus * kMainBlocksPerCU, 3);
  if (sh.seg <= 0) sh.seg = kChunk;
  sh.nseg = (sh.T + sh.seg - 1) / sh.seg;
  sh.nchunk = (sh.T + kChunk - 1) / kChunk;
  sh.ntile = (sh.Di + kBlock - 1) / kBlock;
  const size_t N = dm.d_state, Bt = sh.Bt, Di = sh.Di;
  size_t sz[7] = {0, 0, 0, 0, 0, 0, 0};
  if (bwd && !given_ckpt) {
    sz[0] = Bt * sh.nchunk * N * Di;
    sz[1] = Bt * sh.nchunk * Di;
  }
  sz[2] = given_ckpt ? 0 : Bt * sh.nseg * N * Di;
  sz[3] = bwd ? Bt * sh.nseg * N * Di : 0;
  sz[4] = Bt * sh.nseg * Di;
  if (bwd) {
    sz[5] = (size_t)sh.ntile * Bt * sh.T * 2 * N;
    sz[6] = Bt * sh.nseg * (N + 1) * Di;
  }
  size_t off = 0;
  for (int i = 0; i < 7; ++i) {
    p.off[i] = off;
    off += align_up(sz[i] * sizeof(float));
  }
  p.bytes = off;
  return p;
}

ScanWs bind(const Plan& p, void* ws) {
  char* base = static_cast<char*>(ws);
  ScanWs w;
  w.ckpt = reinterpret_cast<float*>(base + p.off[0]);
  w.ckpt_sd = reinterpret_cast<float*>(base + p.off[1]);
  w.seg_h = reinterpret_cast<float*>(base + p.off[2]);
  w.seg_g = reinterpret_cast<float*>(base + p.off[3]);
  w.seg_sd = reinterpret_cast<float*>(base + p.off[4]);
  w.part_bc = reinterpret_cast<float*>(base + p.off[5]);
  w.part_a = reinterpret_cast<float*>(base + p.off[6]);
  return w;
}

template <typename T, int NS>
int launch_bwd(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
               const float* D, const void* z, const void* d_out, void* d_u, void* d_delta,
               float* d_A_log, void* d_B, void* d_C, float* d_D, void* d_z, int flags,
               const float* h_ckpt, const Plan& p, ScanWs w, hipStream_t st, void* const* ev) {
  auto mark = [&](int k) {
    if (ev && ev[k]) (void)hipEventRecord(static_cast<hipEvent_t>(ev[k]), st);
  };
  const ScanShape& sh = p.sh;
  const T* tu = static_cast<const T*>(u);
  const T* tdl = static_cast<const T*>(delta);
  const T* tB = static_cast<const T*>(B);
  const T* tC = static_cast<const T*>(C);
  const T* tz = static_cast<const T*>(z);
  const T* tdo = static_cast<const T*>(d_out);
  dim3 grid(sh.ntile, sh.nseg, sh.Bt);
  const int ncarry = (int)(((size_t)sh.Bt * NS * sh.Di + kBlock - 1) / kBlock);
  mark(0);
  if (!h_ckpt) {
    hipLaunchKernelGGL((scan_summary<T, NS, true>), grid, dim3(kBlock), 0, st, tu, tdl, A_log, tB, tC, tz, tdo,
                       w.ckpt, w.ckpt_sd, w.seg_h, w.seg_g, w.seg_sd, sh);
    mark(1);
    if (sh.nseg > 1)
      hipLaunchKernelGGL((scan_carry<NS, true, true>), dim3(ncarry), dim3(kBlock), 0, st, A_log, w.seg_h, w.seg_g,
                         w.seg_sd, sh);
  } else {
    if (sh.nseg > 1)
      hipLaunchKernelGGL((scan_gsum<T, NS>), dim3(sh.ntile, sh.nseg - 1, sh.Bt), dim3(kBlock), 0, st, tdl, A_log, tC,
                         tz, tdo, w.seg_g, w.seg_sd, sh);
    mark(1);
    if (sh.nseg > 1)
      hipLaunchKernelGGL((scan_carry<NS, false, true>), dim3(ncarry), dim3(kBlock), 0, st, A_log, w.seg_h, w.seg_g,
                         w.seg_sd, sh);
  }
  mark(2);
  // float sweeps one channel per lane, and so does bf16 from given states;
  // bf16 rebuilding its states sweeps on lane pairs
#define SSM_MAIN(SP, GCK)                                                                                        \
  do {                                                                                                           \
    if constexpr (sizeof(T) == 4 || GCK)                                                                         \
      hipLaunchKernelGGL((scan_bwd_main<T, NS, SP, GCK>), grid, dim3(kBlock), 0, st, tu, tdl, A_log, tB, tC, D, tz, \
                         tdo, static_cast<T*>(d_u), static_cast<T*>(d_delta), static_cast<T*>(d_z),               \
                         GCK ? h_ckpt : w.ckpt, w.ckpt_sd, w.seg_h, w.seg_g, w.part_bc, w.part_a, sh);            \
    else                                                                                                         \
      hipLaunchKernelGGL((scan_bwd_pair<T, NS, SP>), grid, dim3(kBlock), 0, st, tu, tdl, A_log, tB, tC, D, tz,    \
                         tdo, static_cast<T*>(d_u), static_cast<T*>(d_delta), static_cast<T*>(d_z), w.ckpt,       \
                         w.ckpt_sd, w.seg_h, w.seg_g, w.part_bc, w.part_a, sh);                                   \
  } while (0)
  if (h_ckpt) {
    if (flags & SSM_BWD_SOFTPLUS) SSM_MAIN(true, true);
    else SSM_MAIN(false, true);
  } else {
    if (flags & SSM_BWD_SOFTPLUS) SSM_MAIN(true, false);
    else SSM_MAIN(false, false);
  }
#undef SSM_MAIN
  mark(3);
  const size_t nbc = (size_t)sh.Bt * sh.T * 2 * NS;
  const int nblk_bc = (int)((nbc + kBlock - 1) / kBlock);
  const int nblk_a = (NS + 1) * ((sh.Di + kWave - 1) / kWave);
  hipLaunchKernelGGL((scan_bwd_finalize<T, NS>), dim3(nblk_bc + nblk_a), dim3(kBlock), 0, st, A_log,
                     static_cast<T*>(d_B), static_cast<T*>(d_C), d_A_log, d_D, w.part_bc, w.part_a, sh, nblk_bc,
                     (flags & SSM_BWD_ACCUMULATE) ? 1 : 0);
  mark(4);
  return check_launch("ssm_scan_bwd");
}

template <typename T, int NS>
int launch_fwd(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
               const float* D, const void* z, void* y, void* out, float* h_ckpt, int ckpt_every,
               const Plan& p, ScanWs w, hipStream_t st) {
  const ScanShape& sh = p.sh;
  const T* tu = static_cast<const T*>(u);
  const T* tdl = static_cast<const T*>(delta);
  const T* tB = static_cast<const T*>(B);
  const T* tC = static_cast<const T*>(C);
  dim3 grid(sh.ntile, sh.nseg, sh.Bt);
  if (sh.nseg > 1) {
    hipLaunchKernelGGL((scan_summary<T, NS, false>), grid, dim3(kBlock), 0, st, tu, tdl, A_log, tB, tC,
                       (const T*)nullptr, (const T*)nullptr, w.ckpt, w.ckpt_sd, w.seg_h, w.seg_g, w.seg_sd, sh);
    const int nb = (int)(((size_t)sh.Bt * NS * sh.Di + kBlock - 1) / kBlock);
    hipLaunchKernelGGL((scan_carry<NS, true, false>), dim3(nb), dim3(kBlock), 0, st, A_log, w.seg_h, w.seg_g, w.seg_sd, sh);
  }
  const int nckpt = ckpt_every > 0 ? (sh.T + ckpt_every - 1) / ckpt_every : 0;
  hipLaunchKernelGGL((scan_fwd_main<T, NS>), grid, dim3(kBlock), 0, st, tu, tdl, A_log, tB, tC, D,
                     static_cast<const T*>(z), static_cast<T*>(y), static_cast<T*>(out), h_ckpt,
                     ckpt_every > 0 ? ckpt_every : 1, nckpt, w.seg_h, sh);
  return check_launch("ssm_scan_fwd");
}

int zero_params(float* d_A_log, float* d_D, int n_a, int n_d, hipStream_t st) {
  if (n_a > 0) hipLaunchKernelGGL(fill_zero, dim3((n_a + kBlock - 1) / kBlock), dim3(kBlock), 0, st, d_A_log, n_a);
  if (n_d > 0) hipLaunchKernelGGL(fill_zero, dim3((n_d + kBlock - 1) / kBlock), dim3(kBlock), 0, st, d_D, n_d);
  return check_launch("ssm_scan_bwd (empty)");
}

}  // namespace

int scan_check_dims(const ssm_dims* dm, int dtype) { return check_dims(dm, dtype); }

}  // namespace ssm

using namespace ssm;

namespace ssm {
namespace {
// The allocation-free variant of ssm_scan_bwd_ckpt takes its workspace from
// this file-scope device array: one copy per GPU, held until the process ends.
// In host code `scratch` only names the array; its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the device that runs `stream`, which must be
// the current device.
int scratch_address(void* stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(SSM_ERR_LAUNCH, "hipGetDevice failed");
  }
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(SSM_ERR_INVALID_ARG, "the stream's device cannot be queried");
    }
    if (sdev != dev)
      return fail(SSM_ERR_INVALID_ARG, "the stream runs on device %d but device %d is current", sdev, dev);
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(SSM_ERR_UNSUPPORTED, "device index %d above %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(SSM_ERR_LAUNCH, "device address of the static scratch: %s", hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SSM_OK;
}

// use_scratch: the workspace is the static device scratch above (workspace and
// ws_bytes are ignored); the call is rejected if its plan needs more.
int run_bwd(const void* u, const void* delta, const float* A_log, const void* B, const void* C, const float* D,
            const void* z, const void* d_out, const float* h_ckpt, bool ckpt_given, void* d_u, void* d_delta,
            float* d_A_log, void* d_B, void* d_C, float* d_D, void* d_z, int flags, void* workspace,
            size_t ws_bytes, const ssm_dims* dims, int dtype, void* stream, void* const* stage_events,
            bool use_scratch = false) {
  int rc = check_dims(dims, dtype);
  if (rc != SSM_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const ssm_dims dm = *dims;
  const int n_a = dm.d_inner * dm.d_state;
  if (dm.d_inner > 0 && (!A_log || !D || !d_A_log || !d_D))
    return fail(SSM_ERR_INVALID_ARG, "A_log, D, d_A_log and d_D are required");
  if (flags & ~(SSM_BWD_SOFTPLUS | SSM_BWD_ACCUMULATE)) return fail(SSM_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if ((size_t)dm.batch * dm.seqlen * dm.d_inner == 0)  // sums over nothing
    return (flags & SSM_BWD_ACCUMULATE) ? SSM_OK : zero_params(d_A_log, d_D, n_a, dm.d_inner, st);
  if (!u || !delta || !B || !C || !z || !d_out || !d_u || !d_delta || !d_B || !d_C || !d_z)
    return fail(SSM_ERR_INVALID_ARG, "a tensor pointer is null");
  if (ckpt_given && !h_ckpt) return fail(SSM_ERR_INVALID_ARG, "h_ckpt is null");
  if (dtype == SSM_BF16 && !(aligned4(B) && aligned4(C) && aligned4(d_B) && aligned4(d_C)))
    return fail(SSM_ERR_UNSUPPORTED, "bf16 B, C, d_B and d_C must be 4-byte aligned");
  const Plan p = make_plan(dm, dtype, true, ckpt_given);
  if (use_scratch) {
    if (p.bytes > kScratchBytes)
      return fail(SSM_ERR_WORKSPACE, "this shape needs %zu bytes of scratch; the static scratch holds %zu",
                  p.bytes, kScratchBytes);
    rc = scratch_address(stream, &workspace);
    if (rc != SSM_OK) return rc;
    ws_bytes = kScratchBytes;
  }
  if (!workspace || ws_bytes < p.bytes || !aligned256(workspace))
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed (256-byte aligned)",
                workspace ? ws_bytes : 0, p.bytes);
  const ScanWs w = bind(p, workspace);
#define SSM_BWD_CASE(TY, NSV)                                                                                    \
  return launch_bwd<TY, NSV>(u, delta, A_log, B, C, D, z, d_out, d_u, d_delta, d_A_log, d_B, d_C, d_D, d_z, \
                             flags, h_ckpt, p, w, st, stage_events)
  if (dtype == SSM_F32) {
    if (dm.d_state == 16) SSM_BWD_CASE(float, 16);
    if (dm.d_state == 8) SSM_BWD_CASE(float, 8);
    SSM_BWD_CASE(float, 4);
  } else {
    if (dm.d_state == 16) SSM_BWD_CASE(bf16, 16);
    if (dm.d_state == 8) SSM_BWD_CASE(bf16, 8);
    SSM_BWD_CASE(bf16, 4);
  }
#undef SSM_BWD_CASE
}
}  // namespace
}  // namespace ssm

extern "C" size_t ssm_scan_bwd_workspace_size(const ssm_dims* dims, int dtype) {
  if (check_dims(dims, dtype) != SSM_OK) return 0;
  if ((size_t)dims->batch * dims->seqlen * dims->d_inner == 0) return 0;
  return make_plan(*dims, dtype, true).bytes;
}

extern "C" size_t ssm_scan_bwd_ckpt_workspace_size(const ssm_dims* dims, int dtype) {
  if (check_dims(dims, dtype) != SSM_OK) return 0;
  if ((size_t)dims->batch * dims->seqlen * dims->d_inner == 0) return 0;
  return make_plan(*dims, dtype, true, true).bytes;
}

extern "C" size_t ssm_scan_fwd_workspace_size(const ssm_dims* dims, int dtype) {
  if (check_dims(dims, dtype) != SSM_OK) return 0;
  if ((size_t)dims->batch * dims->seqlen * dims->d_inner == 0) return 0;
  return make_plan(*dims, dtype, false).bytes;
}

extern "C" int ssm_scan_bwd(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                            const float* D, const void* z, const void* d_out, void* d_u, void* d_delta,
                            float* d_A_log, void* d_B, void* d_C, float* d_D, void* d_z, int flags,
                            void* workspace, size_t ws_bytes, const ssm_dims* dims, int dtype, void* stream) {
  return run_bwd(u, delta, A_log, B, C, D, z, d_out, nullptr, false, d_u, d_delta, d_A_log, d_B, d_C, d_D, d_z,
                 flags, workspace, ws_bytes, dims, dtype, stream, nullptr);
}

extern "C" int ssm_scan_bwd_timed(const void* u, const void* delta, const float* A_log, const void* B,
                                  const void* C, const float* D, const void* z, const void* d_out, void* d_u,
                                  void* d_delta, float* d_A_log, void* d_B, void* d_C, float* d_D, void* d_z,
                                  int flags, void* workspace, size_t ws_bytes, const ssm_dims* dims,
                                  int dtype, void* stream, void* const* stage_events) {
  return run_bwd(u, delta, A_log, B, C, D, z, d_out, nullptr, false, d_u, d_delta, d_A_log, d_B, d_C, d_D, d_z,
                 flags, workspace, ws_bytes, dims, dtype, stream, stage_events);
}

extern "C" int ssm_scan_bwd_ckpt(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                                 const float* D, const void* z, const void* d_out, const float* h_ckpt, void* d_u,
                                 void* d_delta, float* d_A_log, void* d_B, void* d_C, float* d_D, void* d_z,
                                 int flags, void* workspace, size_t ws_bytes, const ssm_dims* dims,
                                 int dtype, void* stream, void* const* stage_events) {
  return run_bwd(u, delta, A_log, B, C, D, z, d_out, h_ckpt, true, d_u, d_delta, d_A_log, d_B, d_C, d_D, d_z,
                 flags, workspace, ws_bytes, dims, dtype, stream, stage_events);
}

extern "C" size_t ssm_scan_bwd_ckpt_noalloc_capacity(void) { return kScratchBytes; }

extern "C" int ssm_scan_bwd_ckpt_noalloc(const void* u, const void* delta, const float* A_log, const void* B,
                                         const void* C, const float* D, const void* z, const void* d_out,
                                         const float* h_ckpt, void* d_u, void* d_delta, float* d_A_log, void* d_B,
                                         void* d_C, float* d_D, void* d_z, int flags, const ssm_dims* dims,
                                         int dtype, void* stream) {
  return run_bwd(u, delta, A_log, B, C, D, z, d_out, h_ckpt, true, d_u, d_delta, d_A_log, d_B, d_C, d_D, d_z,
                 flags, nullptr, 0, dims, dtype, stream, nullptr, true);
}

extern "C" int ssm_scan_fwd(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                            const float* D, const void* z, void* y, void* out, float* h_ckpt, int ckpt_every,
                            void* workspace, size_t ws_bytes, const ssm_dims* dims, int dtype, void* stream) {
  int rc = check_dims(dims, dtype);
  if (rc != SSM_OK) return rc;
  const ssm_dims dm = *dims;
  if ((size_t)dm.batch * dm.seqlen * dm.d_inner == 0) return SSM_OK;
  if (!u || !delta || !A_log || !B || !C || !D) return fail(SSM_ERR_INVALID_ARG, "an input pointer is null");
  if (out && !z) return fail(SSM_ERR_INVALID_ARG, "out requires z");
  if (h_ckpt && (ckpt_every <= 0 || ckpt_every % kChunk != 0))
    return fail(SSM_ERR_INVALID_ARG, "ckpt_every %d must be a positive multiple of %d", ckpt_every, kChunk);
  if (dtype == SSM_BF16 && !(aligned4(B) && aligned4(C)))
    return fail(SSM_ERR_UNSUPPORTED, "bf16 B and C must be 4-byte aligned");
  const Plan p = make_plan(dm, dtype, false);
  if (!workspace || ws_bytes < p.bytes || !aligned256(workspace))
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed (256-byte aligned)",
                workspace ? ws_bytes : 0, p.bytes);
  const ScanWs w = bind(p, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!h_ckpt) ckpt_every = 0;
#define SSM_FWD_CASE(TY, NSV) \
  return launch_fwd<TY, NSV>(u, delta, A_log, B, C, D, z, y, out, h_ckpt, ckpt_every, p, w, st)
  if (dtype == SSM_F32) {
    if (dm.d_state == 16) SSM_FWD_CASE(float, 16);
    if (dm.d_state == 8) SSM_FWD_CASE(float, 8);
    SSM_FWD_CASE(float, 4);
  } else {
    if (dm.d_state == 16) SSM_FWD_CASE(bf16, 16);
    if (dm.d_state == 8) SSM_FWD_CASE(bf16, 8);
    SSM_FWD_CASE(bf16, 4);
  }
#undef SSM_FWD_CASE
}
