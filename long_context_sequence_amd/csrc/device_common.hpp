// Device-side helpers shared by the gfx950 kernels: vector types, MFMA wrappers, bf16 packing,
// LDS swizzles and the workgroup-to-XCD mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D[32x32] += A[32x16] * B[16x32], bf16 in, fp32 accumulate. Operand layout (checked on gfx950):
// lane l holds A[l%32][8*(l/32) + t] and B[8*(l/32) + t][l%32] for t = 0..7; the accumulator's
// register r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Value of x in the lane 32 positions away combined with x: returns {x[l], x[l^32]} ordered so
// that max/sum of the pair is the same on both lanes.
__device__ __forceinline__ float pair_max(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Row of a 32-row MFMA block whose data a lane loads so that, after the 32x32 product, each
// lane's 8 consecutive accumulator registers map to 8 consecutive keys: swaps bits 2 and 3.
__device__ __forceinline__ int perm_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// 16-byte-chunk swizzles that keep the MFMA operand reads of the LDS tiles bank-conflict free.
// Row-major tile of rows j with C chunks per row (C = 16 for d = 128, 8 for d = 64).
template <int C>
__device__ __forceinline__ int swz_rows(int j) {
  if constexpr (C >= 16) return (j & 3) | ((j & 8) >> 1) | ((j & 4) << 1);
  else return (j & 3) | ((j & 8) >> 1);
}
// Transposed tile (rows n, 8 chunks of 8 keys per row).
__device__ __forceinline__ int swz_t(int n) { return (n & 7) ^ ((n >> 3) & 1); }

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2). Map hardware
// block ids so that consecutive work items land on the same XCD: XCD x runs items
// [x * n/8, (x+1) * n/8). Bijective on [0, n).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int n8 = n & ~7;
  if (bid >= n8) return bid;
  return (bid & 7) * (n8 >> 3) + (bid >> 3);
}

}  // namespace cpa
