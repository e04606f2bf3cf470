// Shared helpers of the gfx950 kernels: storage types, bf16 conversion,
// wave-level shuffles, error reporting for the C entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/ssmbwd.h"

namespace ssm {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bfloat16 storage is a raw 16-bit pattern; conversion is exact on load and
// round-to-nearest-even on store (gfx950's v_cvt_pk_bf16_f32, which also turns
// a NaN into a quiet NaN).
struct bf16 {
  uint16_t bits;
};
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return __uint_as_float(uint32_t(x.bits) << 16); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) {
  return bf16{__builtin_bit_cast(uint16_t, (__bf16)x)};
}
// two values rounded by one instruction: lo in bits 0-15, hi in bits 16-31
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T>
__device__ __forceinline__ float ld(const T* p, size_t i) { return to_f32(p[i]); }
template <typename T>
__device__ __forceinline__ void st(T* p, size_t i, float v) { p[i] = from_f32<T>(v); }

// Row of NS values of a [.., NS] tensor whose address is the same in every lane
// of the wave (B_t, C_t), so the compiler keeps it in scalar registers.
template <int NS>
__device__ __forceinline__ void load_row(const float* __restrict__ p, float (&v)[NS]) {
#pragma unroll
  for (int n = 0; n < NS; ++n) v[n] = p[n];
}
template <int NS>
__device__ __forceinline__ void load_row(const bf16* __restrict__ p, float (&v)[NS]) {
  static_assert(NS % 2 == 0, "bf16 rows are read in pairs");
  const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
  for (int k = 0; k < NS / 2; ++k) {
    uint32_t w = q[k];
    v[2 * k] = __uint_as_float(w << 16);
    v[2 * k + 1] = __uint_as_float(w & 0xffff0000u);
  }
}

// ---- raw buffer access ---------------------------------------------------------
// A gfx9 buffer resource over [base, base + 4 GiB) (no stride; DATA_FORMAT 32 in
// word 3).  A load or store adds a 32-bit per-lane byte offset (VGPR) and a
// wave-uniform byte offset (SGPR) to the base, so no 64-bit per-lane address is
// formed or kept.  The base must be the same in every lane of the wave.
typedef __amdgpu_buffer_rsrc_t BufRes;
__device__ __forceinline__ BufRes buf_res(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}
// element `i` of the lane at wave-uniform byte offset `soff`
template <typename T>
__device__ __forceinline__ float buf_ld(BufRes r, uint32_t i, uint32_t soff);
template <>
__device__ __forceinline__ float buf_ld<float>(BufRes r, uint32_t i, uint32_t soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, i * 4u, soff, 0));
}
template <>
__device__ __forceinline__ float buf_ld<bf16>(BufRes r, uint32_t i, uint32_t soff) {
  return __uint_as_float(uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, i * 2u, soff, 0)) << 16);
}
template <typename T>
__device__ __forceinline__ void buf_st(BufRes r, uint32_t i, uint32_t soff, float v);
template <>
__device__ __forceinline__ void buf_st<float>(BufRes r, uint32_t i, uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, i * 4u, soff, 0);
}
template <>
__device__ __forceinline__ void buf_st<bf16>(BufRes r, uint32_t i, uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(from_f32<bf16>(v).bits, r, i * 2u, soff, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float sigmoid(float x) { return fast_rcp(1.0f + fast_exp2(-x * kLog2e)); }

// ---- cross-lane moves (DPP and the gfx950 permlane swaps) -----------------
// Every control used here (quad_perm, row_ror, row_half_mirror) reads a valid
// lane for every lane, so the "old" value never shows; bound_ctrl lets the
// compiler skip materialising it.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowRor8 = 0x128;        // lane l <- l ^ 8 inside a 16-lane row
constexpr int kRowHalfMirror = 0x141;  // lane l <- 7 - l inside each 8-lane half row

// Wave reduce-scatter of V values per lane (V a power of two, 1..16).  On
// return v[0] of lane l holds the sum over all 64 lanes of the input element
// with index l >> (6 - log2 V) (each result is repeated on 64/V lanes).
// Steps: lane bit 5 and bit 4 halves exchange with permlane32/16 swaps, bits 3
// and 2 with DPP; the bits left once a single value remains are summed with
// DPP butterflies.
template <int V>
__device__ __forceinline__ void wave_reduce_scatter(float (&v)[V], int lane) {
  static_assert(V == 1 || V == 2 || V == 4 || V == 8 || V == 16, "V must be a power of two <= 16");
  if constexpr (V >= 2) {  // lane bit 5
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
      auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + V / 2]),
                                                false, false);
      v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  }
  if constexpr (V >= 4) {  // lane bit 4
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
      auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + V / 4]),
                                                false, false);
      v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  }
  if constexpr (V >= 8) {  // lane bit 3 (partner l ^ 8)
    const bool hi = lane & 8;
#pragma unroll
    for (int i = 0; i < V / 8; ++i) {
      float keep = hi ? v[i + V / 8] : v[i];
      float send = hi ? v[i] : v[i + V / 8];
      v[i] = keep + dpp<kRowRor8>(send);
    }
  }
  if constexpr (V >= 16) {  // lane bit 2 (partner 7 - l within 8; flips bit 2)
    const bool hi = lane & 4;
    float keep = hi ? v[1] : v[0];
    float send = hi ? v[0] : v[1];
    v[0] = keep + dpp<kRowHalfMirror>(send);
  }
  // remaining low bits: all-reduce
  if constexpr (V <= 1) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[0]), false, false);
    v[0] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (V <= 2) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[0]), __float_as_uint(v[0]), false, false);
    v[0] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (V <= 4) v[0] += dpp<kRowRor8>(v[0]);
  if constexpr (V <= 8) v[0] += dpp<kRowHalfMirror>(v[0]);
  v[0] += dpp<kQuadXor1>(v[0]);
  v[0] += dpp<kQuadXor2>(v[0]);
}

// Reduce-scatter of V values per lane (V = 2, 4 or 8) over the 32 lanes that
// share lane bit 0 (the two halves of a lane pair hold different values and are
// never added together).  On return v[0] of lane l holds the sum, over the 32
// lanes with l's bit 0, of the input element with index pair_index<V>(l); the
// lanes with pair_writer<V>(l) hold each such sum once.  Steps: lane bits 5 and
// 4 exchange halves with permlane32/16 swaps, bit 1 (V = 8) with a quad DPP;
// the bits left once a single value remains are summed with DPP rotations
// (row_ror 4 then 8 sums over bits 2 and 3 and leaves bits 0 and 1 alone).
constexpr int kRowRor4 = 0x124;  // lane l <- l + 4 (mod 16) inside a 16-lane row
template <int V>
__device__ __forceinline__ void pair_reduce_scatter(float (&v)[V], int lane) {
  static_assert(V == 2 || V == 4 || V == 8, "V must be 2, 4 or 8");
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {  // lane bit 5
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + V / 2]), false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (V >= 4) {  // lane bit 4
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
      auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + V / 4]), false, false);
      v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  } else {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[0]), __float_as_uint(v[0]), false, false);
    v[0] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (V >= 8) {  // lane bit 1 (partner l ^ 2)
    const bool hi = lane & 2;
    const float keep = hi ? v[1] : v[0];
    const float send = hi ? v[0] : v[1];
    v[0] = keep + dpp<kQuadXor2>(send);
  } else {
    v[0] += dpp<kQuadXor2>(v[0]);
  }
  v[0] += dpp<kRowRor4>(v[0]);
  v[0] += dpp<kRowRor8>(v[0]);
}
template <int V>
__device__ __forceinline__ int pair_index(int lane) {
  return V == 8 ? (((lane >> 3) & 6) | ((lane >> 1) & 1)) : V == 4 ? ((lane >> 4) & 3) : ((lane >> 5) & 1);
}
template <int V>
__device__ __forceinline__ bool pair_writer(int lane) {
  return (lane & (V == 8 ? 0x0C : V == 4 ? 0x0E : 0x1E)) == 0;
}

// ---- error reporting ---------------------------------------------------------
void set_error(const char* fmt, ...);
int fail(int status, const char* fmt, ...);
int check_launch(const char* what);

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// workspaces are carved into 256-byte aligned regions from an aligned base
inline bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

// ---- launchers shared between translation units (arguments already checked) --
// gemm.hip: C = opA * opB on bf16 operands (k contiguous or strided per operand)
size_t gemm_workspace_bytes(int M, int N, int K);
int gemm_check(const void* A, long long lda, const void* B, long long ldb, const void* C, int M, int N, int K,
               size_t ws_bytes, const void* workspace);
int gemm_bf16(const void* A, bool a_kcontig, long long lda, const void* B, bool b_kcontig, long long ldb, void* C,
              long long ldc, int out_dtype, int M, int N, int K, int accumulate, void* workspace, hipStream_t st);
// scan.hip: the scan entry points' argument check (sizes, strides, segment
// length), for callers that must reject a call before their first launch
int scan_check_dims(const ssm_dims* dm, int dtype);
// pointwise.hip: zero fill and the layer's forward pieces
void launch_fill_zero(float* p, int64_t n, hipStream_t st);
void launch_rmsnorm_fwd(const bf16* x, const float* w, bf16* xn, int64_t rows, int dim, float eps, hipStream_t st);
void launch_conv_silu_fwd(const bf16* x, int ld_x, const float* w, const float* bias, bf16* u, int ld_u, int Bt,
                          int Tn, int Di, int K, hipStream_t st);
void launch_gate_fwd(const bf16* y, const bf16* z, int ld_z, bf16* g, int64_t rows, int Di, hipStream_t st);
// (Di a multiple of 8, v 16-byte aligned: the layer's shapes)
void launch_bias_softplus(bf16* v, const float* b, int64_t rows, int Di, hipStream_t st);
void launch_bias_add(bf16* y, const float* b, int64_t rows, int n, hipStream_t st);

}  // namespace ssm
