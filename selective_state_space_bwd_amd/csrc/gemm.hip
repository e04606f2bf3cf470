// bf16 GEMM on the gfx950 matrix cores for the layer's linear layers
// (mamba-rs cpu/backward.rs, the sgemm_backward calls of Phases B1, B4, B5, B7,
// and the matching forward products).
//
//   C[M, N] (+)= sum_k opA(m, k) * opB(k, n),   fp32 accumulation
//   opA(m, k) = A[m * lda + k]  (A_K: k contiguous)  or  A[k * lda + m]
//   opB(k, n) = B[n * ldb + k]  (B_K: k contiguous)  or  B[k * ldb + n]
//
// Two tile families on v_mfma_f32_32x32x16_bf16, both with every operand tile
// in LDS in the layout it has in memory ([row][k] read with ds_read_b128 when k
// is contiguous, [k][row] read with the transposing ds_read_b64_tr_b16
// otherwise):
// - Register-staged tiles (gemm_tile): BM x BN x 32 (256 x 128 for large
//   products, 128 x 128 otherwise), four waves in a 2 x 2 grid, two waves per
//   SIMD, the next tiles' global loads held in registers, edge tiles checked;
//   they take any shape.
// - Direct-load tiles (gemm_big_tile): 256 x 256 or 256 x 128 x 32, one wave
//   per SIMD with the accumulators in AGPRs, operand tiles brought into a ring
//   of LDS stages by global -> LDS loads; they take whole tiles, and the
//   layer's products in pairs (dX and dW of one layer in one launch).
// Split-k writes fp32 partial tiles that a second kernel sums in a fixed order.
#include <math.h>

#include <atomic>

#include "common.hpp"

namespace ssm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 32;
constexpr int kGemmThreads = 256;

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  void* C;          // float or bf16, row stride ldc
  float* partial;   // split-k partials [splits, M, N] (ldc = N), or null
  long long lda, ldb, ldc;
  int M, N, K;
  int k_per_split;  // multiple of kBK
  int accumulate;   // add into C instead of overwriting (the split-k sum adds it)
  int vec_out;      // C rows allow 16-byte vectors (aligned base, ldc a multiple of the vector)
  float* colsum;    // big tiles: sums of A over k per row, [splits, M] with partials (or null)
};

// one 16-byte chunk (8 bf16) of a matrix row, zero outside [0, rows) x [0, cols)
__device__ __forceinline__ uint4 load_chunk(const uint16_t* __restrict__ p, long long ld, int r, int c, int rows,
                                            int cols) {
  uint4 v = make_uint4(0, 0, 0, 0);
  if (r < rows) {
    const uint16_t* q = p + (long long)r * ld + c;
    if (c + 8 <= cols) {
      v = *reinterpret_cast<const uint4*>(q);
    } else {
      uint16_t t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = (c + i < cols) ? q[i] : uint16_t(0);
      v = make_uint4(t[0] | (uint32_t(t[1]) << 16), t[2] | (uint32_t(t[3]) << 16), t[4] | (uint32_t(t[5]) << 16),
                     t[6] | (uint32_t(t[7]) << 16));
    }
  }
  return v;
}

// One operand's R x 32 tile: its global -> register -> LDS moves and its MFMA
// operand reads.
// KC (k contiguous): LDS [row][k], rows of 32 bf16 = four 16-byte chunks, chunk
// c of row r stored at c ^ ((r >> 2) & 3).  The 16 lanes that the 64-bank LDS
// serves together in a 16-byte access then fall in 16 different 16-byte bank
// groups both when a store writes four rows' four chunks and when a fragment
// read takes one chunk of 16 rows (rows 4 apart would otherwise share a group).
// Otherwise: LDS [k][row], rows of R + 32 bf16: the 32 lanes of a transposing
// 8-byte read touch four k rows at two column offsets, and the 64-byte row
// padding puts those eight 32-byte pieces on eight different bank ranges.
template <bool KC, int R>
struct OperandTile {
  static constexpr int kLd = KC ? kBK : R + 32;
  static constexpr int kElems = KC ? R * kLd : kBK * kLd;
  static constexpr int kPer = R * kBK / 8 / kGemmThreads;  // 16-byte chunks per thread
  static_assert(kPer >= 1 && R % 32 == 0, "tile shape");
  uint4 v[kPer];

  static __device__ __forceinline__ int kc_offset(int r, int chunk) {
    return r * kLd + ((chunk ^ ((r >> 2) & 3)) << 3);
  }
  // Interior tiles: each thread's chunks sit at fixed byte offsets from the
  // tile's first element, so a k step only moves a wave-uniform base.
  unsigned off[kPer];
  __device__ __forceinline__ void init(long long ld, int tid) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int c = tid + q * kGemmThreads;
      off[q] = KC ? (unsigned)(((c >> 2) * ld + (c & 3) * 8) * 2)
                  : (unsigned)(((c / (R / 8)) * ld + (c % (R / 8)) * 8) * 2);
    }
  }
  // tile at rows row0.., k k0.., every chunk inside the matrix
  __device__ __forceinline__ void load_full(const uint16_t* __restrict__ base, long long ld, int row0, int k0) {
    const char* t = reinterpret_cast<const char*>(KC ? base + row0 * ld + k0 : base + k0 * ld + row0);
#pragma unroll
    for (int q = 0; q < kPer; ++q) v[q] = *reinterpret_cast<const uint4*>(t + off[q]);
  }
  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, long long ld, int row0, int k0, int rows,
                                       int kend, int tid) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int c = tid + q * kGemmThreads;
      if (KC) {  // R rows x 4 chunks of 8 k
        v[q] = load_chunk(base, ld, row0 + (c >> 2), k0 + (c & 3) * 8, rows, kend);
      } else {   // 32 k rows x R / 8 chunks of 8 tile rows
        v[q] = load_chunk(base, ld, k0 + c / (R / 8), row0 + (c % (R / 8)) * 8, kend, rows);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* __restrict__ lds, int tid) const {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int c = tid + q * kGemmThreads;
      const int off = KC ? kc_offset(c >> 2, c & 3) : (c / (R / 8)) * kLd + (c % (R / 8)) * 8;
      *reinterpret_cast<uint4*>(lds + off) = v[q];
    }
  }
  // MFMA operand of rows rt * 32 .. + 31 and k ks * 16 .. + 15: lane l holds row
  // l % 32 and k 8 (l / 32) .. + 7
  static __device__ __forceinline__ bf16x8_t frag(const uint16_t* __restrict__ lds, int rt, int ks, int lane) {
    if (KC) {
      return *reinterpret_cast<const bf16x8_t*>(&lds[kc_offset(rt * 32 + (lane & 31), ks * 2 + (lane >> 5))]);
    } else {
      // within a 16-lane group, lane i of the transposing read returns element
      // i % 4 of the 8-byte rows addressed by lanes 4r + i / 4, r = 0..3: lane j
      // addresses k row (j / 4) and rows 4 (j % 4) .. + 3, so lane i gets tile row
      // i at four consecutive k
      const int grp = lane >> 4, j = lane & 15;
      const int k = ks * 16 + 8 * (grp >> 1) + (j >> 2);
      const int r = rt * 32 + 16 * (grp & 1) + 4 * (j & 3);
      typedef __attribute__((address_space(3))) v4i16_t lds_v4;
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(lds + k * kLd + r));
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(lds + (k + 4) * kLd + r));
      const v4i16_t lohi[2] = {lo, hi};
      return *reinterpret_cast<const bf16x8_t*>(lohi);
    }
  }
};

constexpr int kStageLd = 36;  // floats per staged row (16-byte aligned rows)

// 16 consecutive outputs of one row starting at column col (< n): 16-byte
// vectors when the row allows it, element by element at the right edge
template <typename T>
__device__ __forceinline__ void write_row16(T* __restrict__ rowp, int col, int n, const float (&v)[16], bool accumulate,
                                            bool vec_ok) {
  constexpr int V = 16 / sizeof(T);  // elements per vector
  if (vec_ok && col + 16 <= n) {
#pragma unroll
    for (int q = 0; q < 16 / V; ++q) {
      T* p = rowp + col + q * V;
      if constexpr (sizeof(T) == 4) {
        float4 o = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        if (accumulate) {
          const float4 prev = *reinterpret_cast<const float4*>(p);
          o.x += prev.x; o.y += prev.y; o.z += prev.z; o.w += prev.w;
        }
        *reinterpret_cast<float4*>(p) = o;
      } else {
        uint4 prev = make_uint4(0, 0, 0, 0);
        if (accumulate) prev = *reinterpret_cast<const uint4*>(p);
        const uint32_t pw[4] = {prev.x, prev.y, prev.z, prev.w};
        uint32_t ow[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float lo = v[8 * q + 2 * e], hi = v[8 * q + 2 * e + 1];
          if (accumulate) {
            lo += __uint_as_float(pw[e] << 16);
            hi += __uint_as_float(pw[e] & 0xffff0000u);
          }
          ow[e] = pack_bf16x2(lo, hi);
        }
        *reinterpret_cast<uint4*>(p) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (col + e < n) {
        T* p = rowp + col + e;
        *p = from_f32<T>((accumulate ? to_f32(*p) : 0.f) + v[e]);
      }
    }
  }
}

// LDS elements of one product's double-buffered A and B tiles; after the k loop
// the same space stages the output tiles (4 waves x 32 rows x kStageLd floats)
template <bool A_K, bool B_K, int BM, int BN>
constexpr int gemm_lds_elems() {
  return 2 * (OperandTile<A_K, BM>::kElems + OperandTile<B_K, BN>::kElems);
}

// Blocks go to the 8 XCDs round-robin by linear id, and each XCD has its own L2:
// when a product's tile count allows, XCD x takes the x-th contiguous run of its
// tiles (row-major, column tiles fastest), so the blocks that share a row tile
// of A run on one XCD.  pid: the block's index among the product's gx x gy
// tiles (of one k split); the caller's linear ids keep pid % 8 = XCD.
__device__ __forceinline__ int xcd_tile(int pid, int ntile) {
  return (ntile % 8 == 0) ? (pid % 8) * (ntile / 8) + pid / 8 : pid;
}

// One output tile of C at rows m0.., columns n0.., over k split `split`.
template <bool A_K, bool B_K, typename OutT, int BM, int BN>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, int m0, int n0, int split, uint16_t* __restrict__ lds) {
  using TA = OperandTile<A_K, BM>;
  using TB = OperandTile<B_K, BN>;
  constexpr int TM = BM / 64, TN = BN / 64;  // 32 x 32 tiles per wave
  static_assert(4 * 32 * kStageLd * 2 <= gemm_lds_elems<A_K, B_K, BM, BN>(),
                "epilogue staging must fit in the tile buffers");
  uint16_t(*lds_a)[TA::kElems] = reinterpret_cast<uint16_t(*)[TA::kElems]>(lds);
  uint16_t(*lds_b)[TB::kElems] = reinterpret_cast<uint16_t(*)[TB::kElems]>(lds + 2 * TA::kElems);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int kb = split * g.k_per_split;
  const int ke = min(g.K, kb + g.k_per_split);
  const int nk = (ke - kb + kBK - 1) / kBK;

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // two register sets carry tiles kt + 1 and kt + 2 while the matrix cores work
  // on tile kt from LDS: the global loads of a tile get two k steps to land
  TA la0, la1;
  TB lb0, lb1;
  // a k step whose whole A and B tiles lie inside the matrices takes unchecked
  // 16-byte loads at fixed per-thread offsets; edge tiles check every element
  const bool interior = m0 + BM <= g.M && n0 + BN <= g.N;
  la0.init(g.lda, tid);
  la1.init(g.lda, tid);
  lb0.init(g.ldb, tid);
  lb1.init(g.ldb, tid);
  const auto load_tile = [&](TA& a, TB& b, int k0) {
    if (interior && k0 + kBK <= ke) {
      a.load_full(g.A, g.lda, m0, k0);
      b.load_full(g.B, g.ldb, n0, k0);
    } else {
      a.load(g.A, g.lda, m0, k0, g.M, ke, tid);
      b.load(g.B, g.ldb, n0, k0, g.N, ke, tid);
    }
  };
  load_tile(la0, lb0, kb);
  if (nk > 1) load_tile(la1, lb1, kb + kBK);
  la0.store(lds_a[0], tid);
  lb0.store(lds_b[0], tid);
  __syncthreads();
  // one k step on LDS buffer `cur`; `nxt_a/b` hold tile kt + 1, `free_a/b` take tile kt + 2
  const auto step = [&](int kt, int cur, TA& free_a, TB& free_b, const TA& nxt_a, const TB& nxt_b) {
    if (kt + 2 < nk) load_tile(free_a, free_b, kb + (kt + 2) * kBK);
    // all operand reads of the k step first, so the second half's reads are in
    // flight while the first half's products run
    bf16x8_t fa[kBK / 16][TM], fb[kBK / 16][TN];
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[ks][i] = TA::frag(lds_a[cur], wm * TM + i, ks, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[ks][j] = TB::frag(lds_b[cur], wn * TN + j, ks, lane);
    }
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks][i], fb[ks][j], acc[i][j], 0, 0, 0);
    if (kt + 1 < nk) {
      nxt_a.store(lds_a[cur ^ 1], tid);
      nxt_b.store(lds_b[cur ^ 1], tid);
    }
    __syncthreads();
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, 0, la0, lb0, la1, lb1);
    if (kt + 1 < nk) step(kt + 1, 1, la1, lb1, la0, lb0);
  }
  // Epilogue.  Accumulator layout of a 32 x 32 tile: register r of lane l holds
  // row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.  Each tile goes through a
  // per-wave LDS area so that lane l then owns row l / 2, columns 16 (l % 2) ..
  // + 15, written (or read, added and written) as 16-byte vectors.
  // the k loop ended with a barrier: no wave reads the tile buffers any more
  float(*stage)[32][kStageLd] = reinterpret_cast<float(*)[32][kStageLd]>(lds);
  float* out_f = g.partial ? g.partial + (long long)split * g.M * g.N : nullptr;
  const long long ldo = g.partial ? g.N : g.ldc;
  const bool vec_ok = g.partial ? (g.N % 4 == 0) : g.vec_out;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) stage[wave][8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)][lane & 31] = acc[i][j][r];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float v[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 t = *reinterpret_cast<const float4*>(&stage[wave][lane >> 1][16 * (lane & 1) + 4 * q]);
        v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
      }
      __builtin_amdgcn_wave_barrier();
      const int row = m0 + (wm * TM + i) * 32 + (lane >> 1);
      const int col = n0 + (wn * TN + j) * 32 + 16 * (lane & 1);
      if (row >= g.M) continue;
      if (out_f) {
        write_row16<float>(out_f + (long long)row * ldo, col, g.N, v, false, vec_ok);
      } else {
        write_row16<OutT>(static_cast<OutT*>(g.C) + (long long)row * ldo, col, g.N, v, g.accumulate != 0, vec_ok);
      }
    }
}

// ---- 256 x BN tiles with direct global -> LDS loads --------------------------
// Block tile 256 x BN (BN 256 or 128), four waves in a 2 x 2 grid, each owning
// a 128 x BN/2 part of it as v_mfma_f32_32x32x16_bf16 tiles (up to 256
// accumulator registers per lane, which the gfx950 register file holds at one
// wave per SIMD).  Operand tiles reach LDS by direct global -> LDS loads
// (global_load_lds_dwordx4: lane i of an instruction writes 16 bytes at the
// instruction's LDS base + 16 i), so no registers stage them; each lane picks
// which 16-byte chunk of the tile it fetches, and that choice sets the LDS
// layout.  Several LDS stages: the loads of tile k + stages - 1 are issued while
// the matrix cores work on tile k, so a load has stages - 1 k steps to arrive;
// the 128-wide tile, used for streaming products with a narrow side, gets six.
// Against the 256 x 128 register-staged tile the 256 x 256 one halves the
// operand bytes per flop and cuts the LDS operand reads per flop by a quarter.
constexpr int kBigT = 256;  // block tile rows (the A side)
constexpr int kBigK = 32;   // k per step

template <int BN>
struct BigCfg {
  static_assert(BN == 256 || BN == 128, "big tile width");
  static constexpr int kNst = BN == 256 ? 4 : 6;                     // LDS stages
  static constexpr int kABytes = kBigT * kBigK * 2;                  // A's tile in one stage
  static constexpr int kBBytes = BN * kBigK * 2;                     // B's tile in one stage
  static constexpr int kStageBytes = kABytes + kBBytes;
  static constexpr int kOnesBytes = BN == 128 ? kBBytes : 0;        // constant B tile for column sums
  static constexpr int kLdsBytes = kNst * kStageBytes + kOnesBytes;  // 128 KB / 152 KB
  static constexpr int kAInst = kABytes / 1024 / 4;                  // direct loads per wave and stage
  static constexpr int kBInst = kBBytes / 1024 / 4;
  static constexpr int kTN = BN / 64;                                // 32-wide n tiles per wave
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

typedef __attribute__((address_space(3))) void* lds_void_t;
typedef __attribute__((address_space(1))) void* gbl_void_t;

// s_waitcnt vmcnt(n), n < 64, and lgkmcnt(0) when `lds` (no wait on the
// export count)
template <int N, bool LDS = false>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070 | (LDS ? 0 : 0x0F00));
}

// One operand's R x 32 tile (R tile rows, 32 k).  Direct load q (0 .. kInst - 1
// over the block) fills LDS bytes [1024 q, 1024 q + 1024) of the operand's area.
// KC (k contiguous): LDS [row][k], 64 bytes per row; 16-byte chunk c of row r
//   sits in slot c ^ ((r >> 2) & 3).  A fragment read takes one chunk of 16
//   consecutive rows per 16 lanes, which then hit 16 different 16-byte bank
//   groups (the row's place in a 256-byte line and the XOR together
//   enumerate them).
// Otherwise: LDS [k][row], 2R bytes per k row; chunk c (8 tile rows) of k row k
//   sits in slot c ^ ((k & 3) << 2).  A transposing read takes four k rows x
//   four chunks per 32 lanes, which land in 16 different bank groups.
template <bool KC, int R>
struct BigOperand {
  static constexpr int kChunksPerRow = KC ? kBigK / 8 : R / 8;  // 16-byte chunks per LDS row
  static constexpr int kRowBytes = kChunksPerRow * 16;
  static constexpr int kRowsPerInst = 1024 / kRowBytes;
  static constexpr int kInst = R * kBigK * 2 / 1024;
  static __device__ __forceinline__ int swz(int row) { return KC ? ((row >> 2) & 3) : ((row & 3) << 2); }
  // Byte offset (from the tile origin) of the chunk that lane `lane` fetches
  // for a direct load of parity `odd`; the rest of the offset is uniform: q x
  // kRowsPerInst x the row stride.  Otherwise-layout tiles with only `valid`
  // rows (a multiple of 8) in the matrix fetch chunk 0 of their k row in place
  // of the chunks past it: the loads stay inside the matrix, and the LDS rows
  // past `valid` hold values that only reach outputs the epilogue drops.
  static __device__ __forceinline__ unsigned lane_src(long long ld, int lane, int odd, int valid) {
    const int row = odd * kRowsPerInst + lane / kChunksPerRow;  // same swizzle as row q * kRowsPerInst + ...
    int c = (lane % kChunksPerRow) ^ swz(row);
    if (!KC && c * 8 >= valid) c = 0;
    return (unsigned)(((lane / kChunksPerRow) * ld + (c << 3)) * 2);
  }
  // the tile origin's element offset in the matrix
  static __device__ __forceinline__ long long origin(long long ld, int row0, int k0) {
    return KC ? (long long)row0 * ld + k0 : (long long)k0 * ld + row0;
  }
  // Per-lane byte offset (inside the operand area) of the MFMA operand of tile
  // rows base + t * 32 .. + 31 at k 16 ks .. + 15; see OperandTile::frag for
  // the lane -> (row, k) map.  KC: one 16-byte read, and t only adds 32 rows,
  // so a lane keeps one offset per ks.  Otherwise: two 8-byte transposing
  // reads, the second 4 k rows further, and ks only adds 16 k rows, so a lane
  // keeps one offset per t.
  static __device__ __forceinline__ unsigned lane_frag(int base, int i, int lane) {
    if (KC) {  // i = ks
      const int r = base + (lane & 31);
      const int c = i * 2 + (lane >> 5);
      return (unsigned)(r * kRowBytes + ((c ^ swz(r)) << 4));
    } else {   // i = t
      const int grp = lane >> 4, j = lane & 15;
      const int k = 8 * (grp >> 1) + (j >> 2);
      const int r = base + i * 32 + 16 * (grp & 1) + 4 * (j & 3);
      return (unsigned)(k * kRowBytes + (((r >> 3) ^ swz(k)) << 4) + (r & 7) * 2);
    }
  }
  static __device__ __forceinline__ bf16x8_t frag(const char* __restrict__ area, const unsigned (&off)[4], int t,
                                                  int ks) {
    if (KC) {
      return *reinterpret_cast<const bf16x8_t*>(area + off[ks] + t * 32 * kRowBytes);
    } else {
      typedef __attribute__((address_space(3))) v4i16_t lds_v4;
      const char* p = area + off[t] + ks * 16 * kRowBytes;
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(p));
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(p + 4 * kRowBytes));
      const v4i16_t lohi[2] = {lo, hi};
      return *reinterpret_cast<const bf16x8_t*>(lohi);
    }
  }
  // value the otherwise-layout byte offset p of a tile holds in the constant
  // tile whose row `one` is 1 and the rest 0 (bf16 bit patterns, as a 16-bit
  // element of the tile's LDS image)
  static __device__ __forceinline__ uint16_t ones_image(int p, int one) {
    const int k = p / kRowBytes, c = ((p % kRowBytes) >> 4) ^ swz(k);
    return (c * 8 + ((p & 15) >> 1)) == one ? uint16_t(0x3F80) : uint16_t(0);
  }
};

// direct load qb (0 .. kInst - 1 over the block) of one operand tile
template <bool KC, int R>
__device__ __forceinline__ void big_load_one(const uint16_t* src, long long ld, char* area, int qb, unsigned off_even,
                                             unsigned off_odd) {
  const char* p = reinterpret_cast<const char*>(src + (long long)qb * BigOperand<KC, R>::kRowsPerInst * ld);
  __builtin_amdgcn_global_load_lds((gbl_void_t)(p + ((qb & 1) ? off_odd : off_even)), (lds_void_t)(area + qb * 1024),
                                   16, 0, 0);
}

// 16 consecutive outputs of one row from a 16-byte aligned column: the big
// tiles' epilogue (rows that take 16-byte vectors)
template <typename T>
__device__ __forceinline__ void write_row16_vec(T* __restrict__ p, const float (&v)[16], bool accumulate) {
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float4 o = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      if (accumulate) {
        const float4 prev = reinterpret_cast<const float4*>(p)[q];
        o.x += prev.x; o.y += prev.y; o.z += prev.z; o.w += prev.w;
      }
      reinterpret_cast<float4*>(p)[q] = o;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint4 prev = make_uint4(0, 0, 0, 0);
      if (accumulate) prev = reinterpret_cast<const uint4*>(p)[q];
      const uint32_t pw[4] = {prev.x, prev.y, prev.z, prev.w};
      uint32_t ow[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float lo = v[8 * q + 2 * e], hi = v[8 * q + 2 * e + 1];
        if (accumulate) {
          lo += __uint_as_float(pw[e] << 16);
          hi += __uint_as_float(pw[e] & 0xffff0000u);
        }
        ow[e] = pack_bf16x2(lo, hi);
      }
      reinterpret_cast<uint4*>(p)[q] = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    }
  }
}

// Block barrier for the big tiles' k loop.  The caller has waited for what the
// other waves must see (its direct loads, through vmcnt); the compiler fences
// keep memory accesses from moving across, and no wait for the direct loads
// still in flight for later stages is implied (a __syncthreads would add one).
__device__ __forceinline__ void big_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 256 x BN output tile at rows m0.., columns n0.., over k split `split`.
// Rows and k are whole tiles and steps (checked by the dispatcher); columns
// may end inside the tile (g.N a multiple of 16, B not k-contiguous).  With
// g.colsum, the B operand's column g.N (past the last output) is taken as all
// ones, so that output column is the sum of A over k: written to
// g.colsum[split * M + row].
template <bool A_K, bool B_K, typename OutT, int BN>
__device__ __forceinline__ void gemm_big_tile(const GemmArgs& g, int m0, int n0, int split, char* __restrict__ lds) {
  using Cfg = BigCfg<BN>;
  using OA = BigOperand<A_K, kBigT>;
  using OB = BigOperand<B_K, BN>;
  constexpr int TN = Cfg::kTN;
  constexpr int kLoads = Cfg::kAInst + Cfg::kBInst;          // per wave and stage
  constexpr int kInFlight = (Cfg::kNst - 2) * kLoads;        // loads of later stages allowed outstanding
  static_assert(kLoads <= 8 && kInFlight < 64, "loads per step");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int kb = split * g.k_per_split;
  const int nk = min(g.k_per_split, g.K - kb) / kBigK;  // whole k steps (checked by the dispatcher)

  floatx16 acc[4][TN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int b_valid = min(BN, g.N - n0);
  const unsigned a_even = OA::lane_src(g.lda, lane, 0, kBigT), a_odd = OA::lane_src(g.lda, lane, 1, kBigT);
  const unsigned b_even = OB::lane_src(g.ldb, lane, 0, b_valid), b_odd = OB::lane_src(g.ldb, lane, 1, b_valid);
  const uint16_t* a0 = g.A + OA::origin(g.lda, m0, kb);
  const uint16_t* b0 = g.B + OB::origin(g.ldb, n0, kb);
  // k step kt's tile origin: KC operands move along the row, the others down k rows
  const long long a_step = A_K ? kBigK : kBigK * g.lda;
  const long long b_step = B_K ? kBigK : kBigK * g.ldb;
  // direct load i (A's loads, then B's) of the wave's share of tile kt (clamped
  // to the last one: the loads past the end refill a stage that nothing reads
  // again) into its stage
  const auto load_one = [&](int kt, int stage, int i) {
    kt = min(kt, nk - 1);
    char* st = lds + stage * Cfg::kStageBytes;
    if (i < Cfg::kAInst)
      big_load_one<A_K, kBigT>(a0 + kt * a_step, g.lda, st, wave * Cfg::kAInst + i, a_even, a_odd);
    else
      big_load_one<B_K, BN>(b0 + kt * b_step, g.ldb, st + Cfg::kABytes, wave * Cfg::kBInst + i - Cfg::kAInst, b_even,
                            b_odd);
  };
  unsigned fa_off[4], fb_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fa_off[i] = OA::lane_frag(wm * 128, i, lane);
    fb_off[i] = OB::lane_frag(wn * (BN / 2), i, lane);
  }
  // the column-sum tile: the n tile of this wave that holds column g.N reads its
  // B operand from the constant tile instead of the stage
  char* ones = lds + Cfg::kNst * Cfg::kStageBytes;
  int ones_t = -1;
  if constexpr (Cfg::kOnesBytes > 0) {
    if (g.colsum) {
      const int t = (g.N - n0 - wn * (BN / 2)) / 32;
      if (g.N - n0 - wn * (BN / 2) >= 0 && t < TN) ones_t = t;
      for (int p = 2 * tid; p < Cfg::kOnesBytes; p += 2 * kGemmThreads)
        *reinterpret_cast<uint16_t*>(ones + p) = OB::ones_image(p, g.N - n0);
    }
  }
  bf16x8_t fa[2][4], fb[2][TN];
  // operand f (0..3: A's row tiles, 4..: B's) of k slice ks into register set `set`
  const auto read_frag = [&](const char* st, int ks, int set, int f) {
    if (f < 4) {
      fa[set][f] = OA::frag(st, fa_off, f, ks);
    } else if (f - 4 < TN) {
      const char* area = (f - 4 == ones_t) ? ones : st + Cfg::kABytes;
      fb[set][f - 4] = OB::frag(area, fb_off, f - 4, ks);
    }
  };
  // A k slice's 4 x TN products as eight fenced chunks, the other register
  // set's reads in the first chunks (two operands each, so every read has at
  // least half the slice to land before its first use) and, with `loads`, one
  // direct load of the step per chunk (spread over the step, not one burst
  // into the address unit).  Without the fences the compiler sinks the reads
  // behind the products to save registers.
  const auto slice = [&](int set, const char* rd_stage, int rd_ks, int load_kt, int load_stage, bool loads) {
    constexpr int P = 4 * TN / 8;  // products per chunk
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (loads && c < kLoads) load_one(load_kt, load_stage, c);
      read_frag(rd_stage, rd_ks, set ^ 1, 2 * c);
      read_frag(rd_stage, rd_ks, set ^ 1, 2 * c + 1);
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const int i = (P * c + e) / TN, j = (P * c + e) % TN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // A bf16 output that is added to: its old values are loaded now, ahead of the
  // first stage's direct loads (so the wait for tile 0 also covers them), and
  // held through the k loop, instead of one dependent load per tile in the
  // epilogue.  Lane: row lane / 2, 16 columns from 16 (lane % 2) of each tile.
  constexpr bool kPrefetch = sizeof(OutT) == 2;
  uint4 prev[4][TN][2];
  const bool prefetch = kPrefetch && !g.partial && g.accumulate;
  if (kPrefetch && prefetch) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const long long row = m0 + wm * 128 + i * 32 + (lane >> 1);
        const int col = n0 + wn * (BN / 2) + j * 32 + 16 * (lane & 1);
        const uint4* q = reinterpret_cast<const uint4*>(static_cast<const OutT*>(g.C) + row * g.ldc + col);
        prev[i][j][0] = col < g.N ? q[0] : make_uint4(0, 0, 0, 0);
        prev[i][j][1] = col < g.N ? q[1] : make_uint4(0, 0, 0, 0);
      }
  }
#pragma unroll
  for (int s = 0; s < Cfg::kNst - 1; ++s)
#pragma unroll
    for (int i = 0; i < kLoads; ++i) load_one(s, s, i);
  wait_vmcnt<kInFlight>();  // tile 0 is in LDS (and so is the constant tile) ...
  __builtin_amdgcn_s_waitcnt(0xC07F);
  big_barrier();            // ... for every wave
#pragma unroll
  for (int f = 0; f < 4 + TN; ++f) read_frag(lds, 0, 0, f);
  // One k step per iteration, with no branch inside, so the accumulators stay
  // in their registers across iterations.  Software pipelined over the two k
  // slices of a step: slice 1's operand reads and the direct loads of tile kt +
  // stages - 1 run under slice 0's products, and after the barrier the next
  // step's slice-0 reads run under slice 1's.  The stage those loads refill was
  // last read before the previous barrier, where every wave arrived only after
  // its own reads had landed.
  int stage = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const int ahead = stage == 0 ? Cfg::kNst - 1 : stage - 1;  // (kt + stages - 1) % stages
    const int next = stage == Cfg::kNst - 1 ? 0 : stage + 1;
    __builtin_amdgcn_sched_barrier(0);
    slice(0, lds + stage * Cfg::kStageBytes, 1, kt + Cfg::kNst - 1, ahead, true);
    // tile kt + 1 is in LDS (later tiles may still be in flight) and this
    // wave's reads of the stage are done; after the barrier, for every wave
    wait_vmcnt<kInFlight, true>();
    big_barrier();
    // (past the last step this reads a stage that nothing uses)
    slice(1, lds + next * Cfg::kStageBytes, 0, 0, 0, false);
    stage = next;
  }
  wait_vmcnt<0, true>();  // the loads past the end and the unused last reads have landed
  big_barrier();           // before LDS is reused
  // Epilogue as in gemm_tile: each 32 x 32 accumulator tile goes through a
  // per-wave LDS area and leaves as rows.
  float(*stage_f)[32][kStageLd] = reinterpret_cast<float(*)[32][kStageLd]>(lds);
  float* out_f = g.partial ? g.partial + (long long)split * g.M * g.N : nullptr;
  const long long ldo = g.partial ? g.N : g.ldc;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) stage_f[wave][8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)][lane & 31] = acc[i][j][r];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float v[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 t = *reinterpret_cast<const float4*>(&stage_f[wave][lane >> 1][16 * (lane & 1) + 4 * q]);
        v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
      }
      __builtin_amdgcn_wave_barrier();
      const long long row = m0 + wm * 128 + i * 32 + (lane >> 1);
      const int col = n0 + wn * (BN / 2) + j * 32 + 16 * (lane & 1);
      if (col < g.N) {
        if (out_f) {
          write_row16_vec<float>(out_f + row * ldo + col, v, false);
        } else if (kPrefetch && prefetch) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const uint32_t pw[4] = {prev[i][j][q].x, prev[i][j][q].y, prev[i][j][q].z, prev[i][j][q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[8 * q + 2 * e] += __uint_as_float(pw[e] << 16);
              v[8 * q + 2 * e + 1] += __uint_as_float(pw[e] & 0xffff0000u);
            }
          }
          write_row16_vec<OutT>(static_cast<OutT*>(g.C) + row * ldo + col, v, false);
        } else {
          write_row16_vec<OutT>(static_cast<OutT*>(g.C) + row * ldo + col, v, g.accumulate != 0);
        }
      } else if (j == ones_t && col == g.N) {
        float* cs = g.colsum + (long long)split * g.M + row;
        *cs = (g.partial || !g.accumulate) ? v[0] : *cs + v[0];
      }
    }
}

// Tile of block pid among ntile tiles (gx columns) for the big tiles: XCD x
// takes the x-th contiguous run of tiles as in xcd_tile, and when the run is
// whole rows of tiles it walks them in groups of four rows, column by column,
// so the blocks an XCD holds at once cover about four row tiles and eight
// column tiles instead of one or two rows of every column.  That roughly
// halves the distinct operand slices the XCD's L2 must hold per k step (a
// wide product's weight was otherwise streamed through every L2 once per
// row of tiles).
__device__ __forceinline__ int grouped_tile(int pid, int ntile, int gx) {
  if (ntile % 8 != 0) return pid;
  const int per = ntile / 8, xcd = pid % 8, local = pid / 8;
  if (per % gx != 0) return xcd * per + local;
  constexpr int G = 4;
  const int nr = per / gx, r0 = xcd * nr;
  const int g = local / (G * gx), gl = min(G, nr - g * G);  // the group's rows
  const int idx = local - g * G * gx;
  return (r0 + g * G + idx % gl) * gx + idx / gl;
}

// grid (column tiles x row tiles x k splits), linear; tiles of one split go
// to the XCDs in contiguous runs (grouped_tile)
template <bool A_K, bool B_K, typename OutT, int BN>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_big_kernel(GemmArgs g, int gx, int ntile) {
  __shared__ __align__(1024) char lds[BigCfg<BN>::kLdsBytes];
  const int split = blockIdx.x / ntile;
  const int tile = grouped_tile(blockIdx.x - split * ntile, ntile, gx);
  gemm_big_tile<A_K, B_K, OutT, BN>(g, (tile / gx) * kBigT, (tile % gx) * BN, split, lds);
}

// Two products in one launch (a linear layer's dX and dW): blocks [0, nb1)
// take product 1's tiles over its k splits (nt1 tiles per split), the rest
// product 2's (nt2 per split)
template <bool A1, bool B1, typename O1, int BN1, bool A2, bool B2, typename O2, int BN2>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_big_pair_kernel(GemmArgs g1, GemmArgs g2, int gx1, int nt1,
                                                                        int nb1, int gx2, int nt2) {
  constexpr int L1 = BigCfg<BN1>::kLdsBytes, L2 = BigCfg<BN2>::kLdsBytes;
  __shared__ __align__(1024) char lds[L1 > L2 ? L1 : L2];
  const int id = blockIdx.x;
  if (id < nb1) {
    const int split = id / nt1;
    const int tile = grouped_tile(id - split * nt1, nt1, gx1);
    gemm_big_tile<A1, B1, O1, BN1>(g1, (tile / gx1) * kBigT, (tile % gx1) * BN1, split, lds);
  } else {
    const int local = id - nb1, split = local / nt2;
    const int tile = grouped_tile(local - split * nt2, nt2, gx2);
    gemm_big_tile<A2, B2, O2, BN2>(g2, (tile / gx2) * kBigT, (tile % gx2) * BN2, split, lds);
  }
}

// grid (column tiles, row tiles, k splits)
template <bool A_K, bool B_K, typename OutT, int BM, int BN>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __align__(16) uint16_t lds[gemm_lds_elems<A_K, B_K, BM, BN>()];
  const int gx = gridDim.x;
  const int tile = xcd_tile(blockIdx.y * gx + blockIdx.x, gx * gridDim.y);
  gemm_tile<A_K, B_K, OutT, BM, BN>(g, (tile / gx) * BM, (tile % gx) * BN, blockIdx.z, lds);
}

// Two independent products in one launch (a linear layer's dX and dW): blocks
// [0, nb1) take product 1's tiles (one k split), the rest product 2's tiles
// over its k splits, so the last round of one product's blocks shares the chip
// with the other's instead of leaving CUs idle.  Both use BM x 128 tiles.
template <bool A1, bool B1, typename O1, bool A2, bool B2, typename O2, int BM>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_pair_kernel(GemmArgs g1, GemmArgs g2, int gx1, int nb1,
                                                                    int gx2, int nt2) {
  constexpr int L1 = gemm_lds_elems<A1, B1, BM, 128>(), L2 = gemm_lds_elems<A2, B2, BM, 128>();
  __shared__ __align__(16) uint16_t lds[L1 > L2 ? L1 : L2];
  const int id = blockIdx.x;
  if (id < nb1) {
    const int tile = xcd_tile(id, nb1);
    gemm_tile<A1, B1, O1, BM, 128>(g1, (tile / gx1) * BM, (tile % gx1) * 128, 0, lds);
  } else {
    const int local = id - nb1, split = local / nt2;
    const int tile = xcd_tile(local - split * nt2, nt2);
    gemm_tile<A2, B2, O2, BM, 128>(g2, (tile / gx2) * BM, (tile % gx2) * 128, split, lds);
  }
}

// Four consecutive outputs of a row per thread (N a multiple of 4: one 16-byte
// load per split), summed over the splits in split order.
template <typename OutT>
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ part, OutT* __restrict__ C,
                                                     long long ldc, int M, int N, int splits, int accumulate) {
  const long long idx = 4 * ((long long)blockIdx.x * 256 + threadIdx.x);
  const long long plane = (long long)M * N;
  if (idx >= plane) return;
  const int row = (int)(idx / N), col = (int)(idx - (long long)row * N);
  float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = 0; s < splits; ++s) {
    const float4 t = *reinterpret_cast<const float4*>(part + s * plane + idx);
    a[0] += t.x; a[1] += t.y; a[2] += t.z; a[3] += t.w;
  }
  OutT* c = C + (long long)row * ldc + col;
#pragma unroll
  for (int e = 0; e < 4; ++e) c[e] = from_f32<OutT>((accumulate ? to_f32(c[e]) : 0.f) + a[e]);
}

// the same for any N, one output per thread
template <typename OutT>
__global__ __launch_bounds__(256) void splitk_reduce1(const float* __restrict__ part, OutT* __restrict__ C,
                                                      long long ldc, int M, int N, int splits, int accumulate) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)M * N) return;
  const int row = (int)(idx / N), col = (int)(idx - (long long)row * N);
  float acc = 0.f;
  for (int s = 0; s < splits; ++s) acc += part[(long long)s * M * N + idx];
  OutT* c = C + (long long)row * ldc + col;
  *c = from_f32<OutT>((accumulate ? to_f32(*c) : 0.f) + acc);
}

// the same for a partial plane [splits, M, N] whose sum lands transposed:
// C[n * ldc + m] (+)= sum_s part[s][m][n], through a 32 x 32 LDS tile so that
// both the partial reads and the output writes are row-contiguous
__global__ __launch_bounds__(256) void splitk_reduce_t(const float* __restrict__ part, float* __restrict__ C,
                                                       long long ldc, int M, int N, int splits, int accumulate) {
  __shared__ float t[32][33];
  const int m0 = blockIdx.x * 32, n0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8 threads
  const long long plane = (long long)M * N;
#pragma unroll
  for (int r = ty; r < 32; r += 8) {
    const int m = m0 + r, n = n0 + tx;
    float a = 0.f;
    if (m < M && n < N)
      for (int s = 0; s < splits; ++s) a += part[s * plane + (long long)m * N + n];
    t[r][tx] = a;
  }
  __syncthreads();
#pragma unroll
  for (int r = ty; r < 32; r += 8) {
    const int n = n0 + r, m = m0 + tx;
    if (m < M && n < N) {
      float* c = C + (long long)n * ldc + m;
      *c = (accumulate ? *c : 0.f) + t[tx][r];
    }
  }
}

// column sums of a [M, N] matrix (bias gradient) in two fixed-order passes:
// block (column tile of 64, row chunk) -> partial[chunk][col], then one sum
// over the chunks per column
constexpr int kColRows = 256;  // rows per chunk

template <typename T>
__global__ __launch_bounds__(256) void column_sum_part(const T* __restrict__ X, long long ldx, int M, int N,
                                                       float* __restrict__ part) {
  __shared__ float s[4][64];
  const int lane = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + lane;
  const int r0 = blockIdx.y * kColRows, r1 = min(M, r0 + kColRows);
  float acc = 0.f;
  if (col < N) {
#pragma unroll 8
    for (int r = r0 + grp; r < r1; r += 4) acc += ld(X, (size_t)r * ldx + col);
  }
  s[grp][lane] = acc;
  __syncthreads();
  if (grp == 0 && col < N) part[(size_t)blockIdx.y * N + col] = s[0][lane] + s[1][lane] + s[2][lane] + s[3][lane];
}

__global__ __launch_bounds__(256) void column_sum_final(const float* __restrict__ part, int chunks, int N,
                                                        float* __restrict__ out, int accumulate) {
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= N) return;
  float acc = 0.f;
#pragma unroll 8
  for (int c = 0; c < chunks; ++c) acc += part[(size_t)c * N + col];
  out[col] = accumulate ? out[col] + acc : acc;
}

namespace {

// CUs of the current device (256 if it cannot be queried), looked up once per device
long gemm_device_cus() {
  static std::atomic<int> cached[64];  // 0 = not looked up yet; every writer stores the same value
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256;
  }
  if (dev >= 0 && dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  if (dev >= 0 && dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Block tile (256 x 128 or 128 x 128 with two or three blocks per CU, or the
// 256 x 256 tile at one block per CU for products made of whole tiles) and k
// splits, picked together from a cost model fitted to measured times of the
// layer's products on the chip: the product's flops at a per-tile-size rate,
// stretched when the last round of blocks leaves CUs idle, plus the split-k
// partial traffic.  256-row tiles need at least 1024 rows and 512 k to pay for
// their set-up; a split keeps at least 128 k.
struct TilePick {
  int bm, splits;
  bool big;
};

// the 256 x 256 tiles take the product: whole tiles in m and n, whole k steps in k
bool big_fits(int M, int N, int K) { return M % kBigT == 0 && N % kBigT == 0 && K % kBigK == 0 && K > 0; }

constexpr double kRate128 = 500e12, kRate256 = 650e12, kRateBig = 1000e12;  // flop/s of the whole chip per tile size

TilePick pick_tiles(int M, int N, int K) {
  static const int kSplits[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32};
  const long cus = gemm_device_cus();
  TilePick best{128, 1, false};
  double best_t = -1.0;
  for (int kind = 0; kind < 3; ++kind) {
    const bool big = kind == 2;
    const int bm = kind == 0 ? 128 : 256, bn = big ? kBigT : 128, kstep = big ? kBigK : kBK;
    if (kind == 1 && (M < 1024 || K < 512)) continue;
    if (big && !big_fits(M, N, K)) continue;
    const double rate = big ? kRateBig : bm == 256 ? kRate256 : kRate128;
    const double slots = (double)cus * (big ? 1 : bm == 256 ? 2 : 3);
    const double tiles = (double)((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    for (int s : kSplits) {
      if (s > 1 && K / s < 4 * kBK) break;
      const int ks = ((K + s - 1) / s + kstep - 1) / kstep * kstep;
      const int used = (K + ks - 1) / ks;  // splits that get k
      const double r = tiles * used / slots, rounds = ceil(r);
      const double work = 2.0 * M * N * K / rate;
      double t = r < 1.0 ? work * rounds / r : work * (1.0 + 0.2 * (rounds - r) / r);
      if (used > 1) t += 2.0 * used * (double)M * N * 4.0 / 3e12;
      if (best_t < 0 || t < best_t) {
        best_t = t;
        best = TilePick{bm, s, big};
      }
    }
  }
  return best;
}

int pick_bm(int M, int N, int K) { return pick_tiles(M, N, K).bm; }
int pick_splits(int M, int N, int K) { return K > 0 ? pick_tiles(M, N, K).splits : 1; }

// k range per split (a multiple of the k step) and the partial buffer; returns the
// number of splits that get k
int gemm_prep(GemmArgs& g, int splits, float* partial, int kstep = kBK) {
  const int ksplit = max(kstep, ((g.K + splits - 1) / splits + kstep - 1) / kstep * kstep);
  g.k_per_split = ksplit;
  const int nsplit = (g.K + ksplit - 1) / ksplit;
  g.partial = nsplit > 1 ? partial : nullptr;
  return nsplit;
}

template <typename OutT>
void gemm_reduce(const GemmArgs& g, int nsplit, float* partial, hipStream_t st) {
  if (nsplit <= 1) return;
  const long long n = (long long)g.M * g.N;
  if (g.N % 4 == 0)  // partial rows are N floats from a 256-byte aligned workspace: 16-byte loads
    hipLaunchKernelGGL((splitk_reduce<OutT>), dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, st, partial,
                       static_cast<OutT*>(g.C), g.ldc, g.M, g.N, nsplit, g.accumulate);
  else
    hipLaunchKernelGGL((splitk_reduce1<OutT>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, partial,
                       static_cast<OutT*>(g.C), g.ldc, g.M, g.N, nsplit, g.accumulate);
}

template <bool A_K, bool B_K, typename OutT>
int launch_gemm(const GemmArgs& g0, int splits, float* partial, hipStream_t st) {
  GemmArgs g = g0;
  const TilePick tp = pick_tiles(g.M, g.N, g.K);
  const int nsplit = gemm_prep(g, splits, partial, tp.big ? kBigK : kBK);
  // the big tiles write 16-byte vectors only: an output they cannot take goes
  // to the 256 x 128 tiles with the same k split
  if (tp.big && (nsplit > 1 || g.vec_out)) {
    const int gx = g.N / kBigT, ntile = gx * (g.M / kBigT);
    hipLaunchKernelGGL((gemm_big_kernel<A_K, B_K, OutT, 256>), dim3((unsigned)(ntile * nsplit)), dim3(kGemmThreads), 0,
                       st, g, gx, ntile);
    gemm_reduce<OutT>(g, nsplit, partial, st);
    return SSM_OK;
  }
  const int bm = tp.big ? 256 : tp.bm;
  dim3 grid((g.N + 127) / 128, (g.M + bm - 1) / bm, nsplit);
  if (bm == 256)
    hipLaunchKernelGGL((gemm_bf16_kernel<A_K, B_K, OutT, 256, 128>), grid, dim3(kGemmThreads), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<A_K, B_K, OutT, 128, 128>), grid, dim3(kGemmThreads), 0, st, g);
  gemm_reduce<OutT>(g, nsplit, partial, st);
  return SSM_OK;
}

}  // namespace

size_t gemm_workspace_bytes(int M, int N, int K) {
  const int s = pick_splits(M, N, K);
  return s > 1 ? align_up((size_t)s * M * N * sizeof(float)) : 0;
}

// argument checks of one product, before anything is launched
int gemm_check(const void* A, long long lda, const void* B, long long ldb, const void* C, int M, int N, int K,
               size_t ws_bytes, const void* workspace) {
  if (M == 0 || N == 0) return SSM_OK;
  if (!A || !B || !C) return fail(SSM_ERR_INVALID_ARG, "gemm: null operand");
  if (!aligned16(A) || !aligned16(B) || (lda & 7) || (ldb & 7))
    return fail(SSM_ERR_UNSUPPORTED, "gemm: operands must be 16-byte aligned with row strides multiple of 8");
  const size_t need = K > 0 ? gemm_workspace_bytes(M, N, K) : 0;
  if (need && (!workspace || ws_bytes < need || !aligned256(workspace)))
    return fail(SSM_ERR_WORKSPACE, "gemm: workspace for split-k missing, too small or not 256-byte aligned");
  return SSM_OK;
}

// C (f32 or bf16 per out_dtype) = opA * opB; see the file comment for the layouts.
// The caller has run gemm_check on the same arguments.
int gemm_bf16(const void* A, bool a_kcontig, long long lda, const void* B, bool b_kcontig, long long ldb, void* C,
              long long ldc, int out_dtype, int M, int N, int K, int accumulate, void* workspace, hipStream_t st) {
  if (M == 0 || N == 0) return SSM_OK;
  const long long vec = out_dtype == SSM_F32 ? 4 : 8;  // elements per 16-byte vector of C
  GemmArgs g{static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), C, nullptr, lda, ldb, ldc, M, N, K,
             0, accumulate, aligned16(C) && ldc % vec == 0};
  const int splits = pick_splits(M, N, K);
  float* part = static_cast<float*>(workspace);
#define GEMM_CASE(AK, BK)                                                                      \
  if (a_kcontig == AK && b_kcontig == BK) {                                                    \
    if (out_dtype == SSM_F32) return launch_gemm<AK, BK, float>(g, splits, part, st);          \
    return launch_gemm<AK, BK, bf16>(g, splits, part, st);                                     \
  }
  GEMM_CASE(true, true)
  GEMM_CASE(true, false)
  GEMM_CASE(false, true)
  GEMM_CASE(false, false)
#undef GEMM_CASE
  return fail(SSM_ERR_INVALID_ARG, "gemm: layout");
}

// Finish time, in k steps, of n1 blocks of d1 k steps followed by n2 blocks of d2
// on `slots` block slots, each block starting on the earliest free slot in
// launch order (the dispatcher's order).  Slots that free together stay one
// group, so the walk takes a few steps per round.
double pair_makespan(long slots, long n1, double d1, long n2, double d2) {
  struct Group { double t; long n; };
  Group g[64];
  int ng = 1;
  g[0] = Group{0.0, slots};
  double end = 0.0;
  long left[2] = {n1, n2};
  const double dur[2] = {d1, d2};
  for (int p = 0; p < 2; ++p) {
    while (left[p] > 0) {
      int e = 0;  // earliest free group
      for (int i = 1; i < ng; ++i)
        if (g[i].t < g[e].t) e = i;
      const long take = left[p] < g[e].n ? left[p] : g[e].n;
      const double t = g[e].t + dur[p];
      end = t > end ? t : end;
      left[p] -= take;
      g[e].n -= take;
      if (g[e].n == 0) g[e] = g[--ng];
      int m = -1;
      for (int i = 0; i < ng; ++i)
        if (g[i].t == t) m = i;
      if (m >= 0) g[m].n += take;
      else if (ng < 64) g[ng++] = Group{t, take};
      else return -1.0;  // more than 64 distinct free times: the caller skips this split
    }
  }
  return end;
}

// dW's k split in the paired launch of linear_bwd_products (splits 0: the
// products are not paired), for an m x N output gradient and an N x K weight.
// With big tiles when both products are made of whole 256 x 256 tiles and
// 32-wide k steps; otherwise the products pair when dX needs no k split and
// both pick the same tile height.  The split is picked for the two products'
// blocks together: the modelled finish time of the block schedule (a k step
// per block costing the same in both, a fixed set-up per block, the tile rate
// of the single-product model) plus the split-k partial traffic.  Big tiles
// also try dW's blocks first: its long blocks then start together and dX's
// short ones fill in behind them.
struct PairPick {
  int splits;
  bool big;
  bool dw_first;
};
constexpr double kSplitSumLaunch = 20e-6;

PairPick pair_dw_splits(int m, int K, int N) {
  const bool big = big_fits(m, K, N) && big_fits(N, K, m);
  const int bm = big ? kBigT : pick_bm(m, K, N), bn = big ? kBigT : 128;
  const int kstep = big ? kBigK : kBK;
  if (!big && (pick_splits(m, K, N) != 1 || pick_bm(N, K, m) != bm)) return PairPick{0, false, false};
  const int gx = (K + bn - 1) / bn;
  const long nb1 = (long)gx * ((m + bm - 1) / bm), nt2 = (long)gx * ((N + bm - 1) / bm);
  const long slots = gemm_device_cus() * (big ? 1 : bm == 256 ? 2 : 3);
  const double rate = big ? kRateBig : bm == 256 ? kRate256 : kRate128;
  const double kstep_s = (double)bm * bn * kstep * 2 / (rate / slots);
  const double setup = big ? 6.0 : 8.0;  // k steps' worth of prologue and epilogue per block
  PairPick best{big ? 1 : pick_splits(N, K, m), big, false};
  double best_t = -1.0;
  for (int order = 0; order < (big ? 2 : 1); ++order) {
    for (int sp : {1, 2, 3, 4, 6, 8, 12, 16, 24, 32}) {
      if (sp > 1 && m / sp < 4 * kBK) break;
      const int ks = ((m + sp - 1) / sp + kstep - 1) / kstep * kstep;
      const int used = (m + ks - 1) / ks;
      const double d1 = (N + kstep - 1) / kstep + setup, d2 = ks / kstep + setup;
      const double ms = order == 0 ? pair_makespan(slots, nb1, d1, nt2 * used, d2)
                                   : pair_makespan(slots, nt2 * used, d2, nb1, d1);
      if (ms < 0) continue;
      double t = ms * kstep_s;
      // a k split adds its partials' traffic and the split-k sum's own launch,
      // which starts only after the pair's last block (20 us in the model's
      // units, fitted to the measured order of the layer's in_proj and out_proj
      // plans: in_proj 0.529 ms unsplit against 0.558 ms with two dW splits)
      if (used > 1) t += 2.0 * used * (double)N * K * 4.0 / 3e12 + kSplitSumLaunch;
      if (best_t < 0 || t < best_t) {
        best_t = t;
        best = PairPick{sp, big, order == 1};
      }
    }
  }
  return best;
}

// Both products of a linear layer whose input width K is narrow (at most 128,
// a multiple of 16: dt_proj's rank) over many rows m and a wide output N, on
// 256 x 128 tiles in one launch: dX [m, K] over k = N and dW [N, K] over k =
// m, each split over k, every block streaming a 256 x 32 slice of dY per step.
// The bias gradient rides along as dW's column K (a column of ones in X) when K
// < 128.  Splits are picked for the two products' blocks together, one block
// per CU: the modelled finish time of the block schedule, in k steps of equal
// cost, plus the split-k partial traffic.
struct SkinnyPlan {
  int s1, s2;   // k splits of dX and dW (0: the shape does not take this path)
  bool colsum;  // db as dW's extra column
};

SkinnyPlan skinny_plan(int m, int K, int N, bool need_db) {
  SkinnyPlan p{0, 0, false};
  if (K > 128 || K % 16 || m % kBigT || N % kBigT || m < 4 * kBigK || N < 4 * kBigK) return p;
  const long slots = gemm_device_cus();
  const double step_s = 1.3e-6;  // one k step of every CU's block, streaming 24 KB each
  double best_t = -1.0;
  for (int s1 : {1, 2, 3, 4, 6, 8}) {
    const int ks1 = ((N + s1 - 1) / s1 + kBigK - 1) / kBigK * kBigK;
    if ((N + ks1 - 1) / ks1 != s1) continue;
    for (int s2 = 1; s2 <= 32; ++s2) {
      const int ks2 = ((m + s2 - 1) / s2 + kBigK - 1) / kBigK * kBigK;
      if ((m + ks2 - 1) / ks2 != s2) continue;
      const long n1 = (long)(m / kBigT) * s1, n2 = (long)(N / kBigT) * s2;
      const double ms = pair_makespan(slots, n1, ks1 / kBigK + 4.0, n2, ks2 / kBigK + 4.0);
      if (ms < 0) continue;
      const double part = (s1 > 1 ? (double)s1 * m * K : 0.0) + (s2 > 1 ? (double)s2 * N * K : 0.0);
      const double t = ms * step_s + 2.0 * part * 4.0 / 3e12;
      if (best_t < 0 || t < best_t) {
        best_t = t;
        p = SkinnyPlan{s1, s2, need_db && K < 128};
      }
    }
  }
  return p;
}

// the skinny plan for these operands: a product written without a k split
// needs 16-byte vectors in its output rows
SkinnyPlan skinny_plan_for(int m, int K, int N, bool need_db, const void* dX, long long lddx, const void* dW) {
  SkinnyPlan p = skinny_plan(m, K, N, need_db);
  if (p.s1 && ((p.s1 == 1 && !(aligned16(dX) && lddx % 8 == 0)) || (p.s2 == 1 && !aligned16(dW))))
    p = SkinnyPlan{0, 0, false};
  return p;
}

// workspace of the skinny pair: dX partials, dW partials, db partials
size_t skinny_workspace_bytes(const SkinnyPlan& p, int m, int K, int N) {
  if (!p.s1) return 0;
  return (p.s1 > 1 ? align_up((size_t)p.s1 * m * K * 4) : 0) + (p.s2 > 1 ? align_up((size_t)p.s2 * N * K * 4) : 0) +
         (p.colsum ? align_up((size_t)p.s2 * N * 4) : 0);
}

void launch_skinny_pair(const SkinnyPlan& p, const void* X, long long ldx, const void* W, const void* dY,
                        long long lddy, void* dX, long long lddx, float* dW, float* db, int m, int K, int N, int acc_x,
                        int acc_w, void* workspace, hipStream_t st) {
  char* ws = static_cast<char*>(workspace);
  float* part1 = nullptr;
  float* part2 = nullptr;
  float* part_db = nullptr;
  if (p.s1 > 1) { part1 = reinterpret_cast<float*>(ws); ws += align_up((size_t)p.s1 * m * K * 4); }
  if (p.s2 > 1) { part2 = reinterpret_cast<float*>(ws); ws += align_up((size_t)p.s2 * N * K * 4); }
  if (p.colsum) part_db = reinterpret_cast<float*>(ws);
  const uint16_t* y16 = static_cast<const uint16_t*>(dY);
  // dX[m, K] = dY[m, N] W[N, K]: A = dY (k = n contiguous), B(k = n, j) = W[n * K + j]
  GemmArgs g1{y16, static_cast<const uint16_t*>(W), dX, nullptr, lddy, K, lddx, m, K, N, 0, acc_x,
              aligned16(dX) && lddx % 8 == 0, nullptr};
  // dW[N, K] = dY^T X: A(i = n, k = row) = dY[row * lddy + n], B(k = row, j) = X[row * ldx + j]
  GemmArgs g2{y16, static_cast<const uint16_t*>(X), dW, nullptr, lddy, ldx, K, N, K, m, 0, acc_w,
              aligned16(dW) && K % 4 == 0, nullptr};
  const int ns1 = gemm_prep(g1, p.s1, part1, kBigK), ns2 = gemm_prep(g2, p.s2, part2, kBigK);
  if (p.colsum) g2.colsum = p.s2 > 1 ? part_db : db;
  const int nt1 = m / kBigT, nt2 = N / kBigT;
  hipLaunchKernelGGL((gemm_big_pair_kernel<true, false, bf16, 128, false, false, float, 128>),
                     dim3((unsigned)(nt1 * ns1 + nt2 * ns2)), dim3(kGemmThreads), 0, st, g1, g2, 1, nt1, nt1 * ns1, 1,
                     nt2);
  gemm_reduce<bf16>(g1, ns1, part1, st);
  gemm_reduce<float>(g2, ns2, part2, st);
  if (p.colsum && ns2 > 1)
    hipLaunchKernelGGL(column_sum_final, dim3((N + 255) / 256), dim3(256), 0, st, part_db, ns2, N, db, acc_w);
}

// Both products of a linear layer with a narrow output N (at most 128, a
// multiple of 32: x_proj) over many rows m and a wide input K, in one launch:
// dW's transpose [K, N] = X^T dY on 256 x 128 tiles split over k = m (its
// partials summed into dW transposed), and dX [m, K] = dY W on 256 x 256
// tiles with its 32 k steps.  dW's long blocks come first and dX's short ones
// fill in behind them.  The split is picked for the two products' blocks
// together: the modelled finish time of the block schedule (a dX block costing
// its k steps plus 8 for the read-modify-write of its tile) plus the partial
// traffic.
int wide_plan(int m, int K, int N, const void* dX, long long lddx) {
  if (N > 128 || N % 32 || m % kBigT || K % kBigT || m < 8 * kBigK || !(aligned16(dX) && lddx % 8 == 0)) return 0;
  const long slots = gemm_device_cus();
  const double step_s = 1.3e-6;
  const long n2 = (long)(m / kBigT) * (K / kBigT);
  int best = 0;
  double best_t = -1.0;
  for (int s1 = 2; s1 <= 32; ++s1) {
    const int ks1 = ((m + s1 - 1) / s1 + kBigK - 1) / kBigK * kBigK;
    if ((m + ks1 - 1) / ks1 != s1) continue;
    const long n1 = (long)(K / kBigT) * s1;
    const double ms = pair_makespan(slots, n1, ks1 / kBigK + 4.0, n2, N / kBigK + 8.0);
    if (ms < 0) continue;
    const double t = ms * step_s + 2.0 * s1 * (double)K * N * 4.0 / 3e12;
    if (best_t < 0 || t < best_t) {
      best_t = t;
      best = s1;
    }
  }
  return best;
}

size_t wide_workspace_bytes(int s1, int K, int N) { return s1 ? align_up((size_t)s1 * K * N * 4) : 0; }

void launch_wide_pair(int s1, const void* X, long long ldx, const void* W, const void* dY, long long lddy, void* dX,
                      long long lddx, float* dW, int m, int K, int N, int acc_x, int acc_w, void* workspace,
                      hipStream_t st) {
  float* part = static_cast<float*>(workspace);
  // dW^T[K, N] = X^T dY: A(i = j, k = row) = X[row * ldx + j], B(k = row, n) = dY[row * lddy + n]
  GemmArgs g1{static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(dY), nullptr, nullptr, ldx, lddy, N,
              K, N, m, 0, 0, 1, nullptr};
  // dX[m, K] = dY[m, N] W[N, K]: A = dY (k = n contiguous), B(k = n, j) = W[n * K + j]
  GemmArgs g2{static_cast<const uint16_t*>(dY), static_cast<const uint16_t*>(W), dX, nullptr, lddy, K, lddx, m, K, N,
              0, acc_x, 1, nullptr};
  const int ns1 = gemm_prep(g1, s1, part, kBigK);
  gemm_prep(g2, 1, nullptr, kBigK);
  g1.partial = part;  // always through partials: the sum lands transposed
  const int nt1 = K / kBigT, gx2 = K / kBigT, nt2 = gx2 * (m / kBigT);
  hipLaunchKernelGGL((gemm_big_pair_kernel<false, false, float, 128, true, false, bf16, 256>),
                     dim3((unsigned)(nt1 * ns1 + nt2)), dim3(kGemmThreads), 0, st, g1, g2, 1, nt1, nt1 * ns1, gx2,
                     nt2);
  hipLaunchKernelGGL(splitk_reduce_t, dim3((K + 31) / 32, (N + 31) / 32), dim3(256), 0, st, part, dW, (long long)K,
                     K, N, ns1, acc_w);
}

// dX[M, K] = dY W and dW[N, K] = dY^T X of one linear layer: one launch for both
// when pair_dw_splits allows (dW's split-k partials then own the workspace),
// otherwise one launch each.
void linear_bwd_products(const void* X, long long ldx, const void* W, const void* dY, long long lddy, void* dX,
                         long long lddx, float* dW, int m, int K, int N, int acc_x, int acc_w, void* workspace,
                         hipStream_t st) {
  PairPick pp = (dX && dW) ? pair_dw_splits(m, K, N) : PairPick{0, false, false};
  // the big tiles write 16-byte vectors only (dW's partials always take them)
  if (pp.big && !((aligned16(dX) && lddx % 8 == 0) && (pp.splits > 1 || aligned16(dW)))) pp.splits = 0;
  if (pp.splits == 0) {
    if (dX) gemm_bf16(dY, true, lddy, W, false, K, dX, lddx, SSM_BF16, m, K, N, acc_x, workspace, st);
    if (dW) gemm_bf16(dY, false, lddy, X, false, ldx, dW, K, SSM_F32, N, K, m, acc_w, workspace, st);
    return;
  }
  const uint16_t* y16 = static_cast<const uint16_t*>(dY);
  GemmArgs g1{y16, static_cast<const uint16_t*>(W), dX, nullptr, lddy, K, lddx, m, K, N, 0, acc_x,
              aligned16(dX) && lddx % 8 == 0};
  GemmArgs g2{y16, static_cast<const uint16_t*>(X), dW, nullptr, lddy, ldx, K, N, K, m, 0, acc_w,
              aligned16(dW) && K % 4 == 0};
  float* part = static_cast<float*>(workspace);
  const int kstep = pp.big ? kBigK : kBK;
  gemm_prep(g1, 1, nullptr, kstep);
  const int nsplit2 = gemm_prep(g2, pp.splits, part, kstep);
  if (pp.big && pp.dw_first) {
    const int gx = K / kBigT, nt1 = gx * (N / kBigT), nt2 = gx * (m / kBigT);
    hipLaunchKernelGGL((gemm_big_pair_kernel<false, false, float, 256, true, false, bf16, 256>),
                       dim3((unsigned)(nt1 * nsplit2 + nt2)), dim3(kGemmThreads), 0, st, g2, g1, gx, nt1,
                       nt1 * nsplit2, gx, nt2);
  } else if (pp.big) {
    const int gx = K / kBigT, nb1 = gx * (m / kBigT), nt2 = gx * (N / kBigT);
    hipLaunchKernelGGL((gemm_big_pair_kernel<true, false, bf16, 256, false, false, float, 256>),
                       dim3((unsigned)(nb1 + nt2 * nsplit2)), dim3(kGemmThreads), 0, st, g1, g2, gx, nb1, nb1, gx, nt2);
  } else {
    const int bm = pick_bm(m, K, N);
    const int gx = (K + 127) / 128;
    const int nb1 = gx * ((m + bm - 1) / bm), nt2 = gx * ((N + bm - 1) / bm);
    const dim3 grid((unsigned)(nb1 + nt2 * nsplit2));
    if (bm == 256)
      hipLaunchKernelGGL((gemm_pair_kernel<true, false, bf16, false, false, float, 256>), grid, dim3(kGemmThreads),
                         0, st, g1, g2, gx, nb1, gx, nt2);
    else
      hipLaunchKernelGGL((gemm_pair_kernel<true, false, bf16, false, false, float, 128>), grid, dim3(kGemmThreads),
                         0, st, g1, g2, gx, nb1, gx, nt2);
  }
  gemm_reduce<float>(g2, nsplit2, part, st);
}

size_t column_sum_workspace_bytes(int M, int N) {
  return align_up((size_t)((M + kColRows - 1) / kColRows) * N * sizeof(float));
}

// workspace: column_sum_workspace_bytes(M, N)
int column_sum_launch(const void* X, long long ldx, int M, int N, int dtype, float* out, int accumulate,
                      void* workspace, hipStream_t st) {
  const int chunks = (M + kColRows - 1) / kColRows;
  float* part = static_cast<float*>(workspace);
  const dim3 grid((N + 63) / 64, chunks);
  if (dtype == SSM_F32)
    hipLaunchKernelGGL(column_sum_part<float>, grid, dim3(256), 0, st, static_cast<const float*>(X), ldx, M, N, part);
  else
    hipLaunchKernelGGL(column_sum_part<bf16>, grid, dim3(256), 0, st, static_cast<const bf16*>(X), ldx, M, N, part);
  hipLaunchKernelGGL(column_sum_final, dim3((N + 255) / 256), dim3(256), 0, st, part, chunks, N, out, accumulate);
  return SSM_OK;
}

}  // namespace ssm

using namespace ssm;

extern "C" size_t linear_bwd_workspace_size(int64_t M, int K, int N) {
  if (M <= 0 || K <= 0 || N <= 0 || M >= (1LL << 31)) return 0;
  // dX = dY W (M x K, reduction N), dW = dY^T X (N x K, reduction M) and the db
  // column sums run one after another and share the space
  size_t a = gemm_workspace_bytes((int)M, K, N), b = gemm_workspace_bytes(N, K, (int)M);
  const size_t sk = skinny_workspace_bytes(skinny_plan((int)M, K, N, true), (int)M, K, N);  // both products at once
  a = sk > a ? sk : a;
  // the wide pair's plan with an aligned dX (a dX it cannot take runs the other paths)
  const size_t wd = wide_workspace_bytes(wide_plan((int)M, K, N, reinterpret_cast<const void*>(256), 8), K, N);
  a = wd > a ? wd : a;
  const int s2 = pair_dw_splits((int)M, K, N).splits;  // dW's split when paired with dX
  if (s2 > 1) {
    const size_t bp = align_up((size_t)s2 * N * K * sizeof(float));
    b = bp > b ? bp : b;
  }
  const size_t c = column_sum_workspace_bytes((int)M, N);
  return a > b ? (a > c ? a : c) : (b > c ? b : c);
}

extern "C" int linear_bwd(const void* X, int64_t ldx, const void* W, const void* dY, int64_t lddy, void* dX,
                          int64_t lddx, int flags, float* dW, float* db, int64_t M, int K, int N,
                          void* workspace, size_t ws_bytes, int dtype, void* stream) {
  if (dtype != SSM_BF16) return fail(SSM_ERR_UNSUPPORTED, "linear_bwd runs on bf16 operands");
  if (flags & ~(SSM_BWD_ACCUMULATE | SSM_BWD_ACCUMULATE_DX)) return fail(SSM_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (M < 0 || K <= 0 || N <= 0 || M >= (1LL << 31))
    return fail(SSM_ERR_INVALID_ARG, "bad size (M %lld K %d N %d)", (long long)M, K, N);
  if ((dW && ldx < K) || lddy < N || (dX && lddx < K)) return fail(SSM_ERR_INVALID_ARG, "row strides below the row length");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int acc_w = (flags & SSM_BWD_ACCUMULATE) ? 1 : 0, acc_x = (flags & SSM_BWD_ACCUMULATE_DX) ? 1 : 0;
  if (M == 0) {  // dX is empty; dW and db are sums over no rows
    if (acc_w || (!dW && !db)) return SSM_OK;
    if (dW) launch_fill_zero(dW, (int64_t)N * K, st);
    if (db) launch_fill_zero(db, N, st);
    return check_launch("linear_bwd (no rows)");
  }
  if (!W || !dY || (dW && !X)) return fail(SSM_ERR_INVALID_ARG, "a tensor pointer is null");
  const int m = (int)M;
  int rc = SSM_OK;
  // dX[M, K] = dY[M, N] W[N, K]: A = dY (k = n contiguous), B(k = n, j) = W[n * K + j]
  if (dX && (rc = gemm_check(dY, lddy, W, K, dX, m, K, N, ws_bytes, workspace)) != SSM_OK) return rc;
  // dW[N, K] = dY^T X: A(i = n, k = m) = dY[m * lddy + n], B(k = m, j) = X[m * ldx + j]
  if (dW && (rc = gemm_check(dY, lddy, X, ldx, dW, N, K, m, ws_bytes, workspace)) != SSM_OK) return rc;
  const SkinnyPlan sp = (dX && dW) ? skinny_plan_for(m, K, N, db != nullptr, dX, lddx, dW) : SkinnyPlan{0, 0, false};
  const int wp = (dX && dW && !sp.s1) ? wide_plan(m, K, N, dX, lddx) : 0;
  const size_t sk = skinny_workspace_bytes(sp, m, K, N) + wide_workspace_bytes(wp, K, N);
  if (sk && (!workspace || ws_bytes < sk || !aligned256(workspace)))
    return fail(SSM_ERR_WORKSPACE, "linear_bwd: workspace for the split-k partials missing, too small or not "
                                   "256-byte aligned");
  if (dX && dW && !sp.s1 && !wp) {  // dX and dW in one launch: dW's split-k partials for the paired split
    const int s2 = pair_dw_splits(m, K, N).splits;
    if (s2 > 1 && (!workspace || ws_bytes < align_up((size_t)s2 * N * K * sizeof(float)) || !aligned256(workspace)))
      return fail(SSM_ERR_WORKSPACE, "linear_bwd: workspace for the split-k partials missing, too small or not "
                                     "256-byte aligned");
  }
  if (db && (!workspace || ws_bytes < column_sum_workspace_bytes(m, N) || !aligned256(workspace)))
    return fail(SSM_ERR_WORKSPACE, "linear_bwd: workspace for the bias sums missing, too small or not 256-byte aligned");
  if (sp.s1)
    launch_skinny_pair(sp, X, ldx, W, dY, lddy, dX, lddx, dW, db, m, K, N, acc_x, acc_w, workspace, st);
  else if (wp)
    launch_wide_pair(wp, X, ldx, W, dY, lddy, dX, lddx, dW, m, K, N, acc_x, acc_w, workspace, st);
  else
    linear_bwd_products(X, ldx, W, dY, lddy, dX, lddx, dW, m, K, N, acc_x, acc_w, workspace, st);
  if (db && !sp.colsum) column_sum_launch(dY, lddy, m, N, SSM_BF16, db, acc_w, workspace, st);
  return check_launch("linear_bwd");
}

extern "C" int linear_fwd(const void* X, int64_t ldx, const void* W, const float* bias, void* Y, int64_t ldy,
                          int64_t M, int K, int N, void* workspace, size_t ws_bytes, int dtype, void* stream) {
  if (dtype != SSM_BF16) return fail(SSM_ERR_UNSUPPORTED, "linear_fwd runs on bf16 operands");
  if (M < 0 || M >= (1LL << 31) || K <= 0 || N <= 0 || ldx < K || ldy < N) return fail(SSM_ERR_INVALID_ARG, "bad size or stride");
  if (!X || !W || !Y) return fail(SSM_ERR_INVALID_ARG, "a tensor pointer is null");
  if (bias) return fail(SSM_ERR_UNSUPPORTED, "linear_fwd bias is applied by the caller's epilogue");
  // Y[M, N] = X[M, K] W[N, K]^T: both operands k-contiguous
  const int rc = gemm_check(X, ldx, W, K, Y, (int)M, N, K, ws_bytes, workspace);
  if (rc != SSM_OK) return rc;
  gemm_bf16(X, true, ldx, W, true, K, Y, ldy, SSM_BF16, (int)M, N, K, 0, workspace, static_cast<hipStream_t>(stream));
  return check_launch("linear_fwd");
}

extern "C" size_t linear_fwd_workspace_size(int64_t M, int K, int N) {
  if (M <= 0 || K <= 0 || N <= 0 || M >= (1LL << 31)) return 0;
  return gemm_workspace_bytes((int)M, N, K);
}
