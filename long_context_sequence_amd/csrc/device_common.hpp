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

// Row-major bf16 tile of D columns in LDS. Its 16-byte chunks are XOR-swizzled per row so that
// both the row reads (8 consecutive columns of rows perm_row(l%32)) and the transposed reads
// (one column of 4 consecutive rows per 16-lane group) spread over all banks.
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  if constexpr (D >= 128) return ((r & 3) << 1) | ((r >> 3) & 1) | (((r >> 2) & 1) << 3);
  else return ((r & 3) << 1) | ((r >> 3) & 1);
}
// Element offset of 16-byte chunk `chunk` (columns 8*chunk .. 8*chunk+7) of row r.
template <int D>
__device__ __forceinline__ int tile_off(int r, int chunk) {
  return r * D + 8 * (chunk ^ tile_swz<D>(r));
}
// Row operand: columns [8*chunk, 8*chunk + 8) of row r.
template <int D>
__device__ __forceinline__ u32x4_t tile_row8(const uint16_t* t, int r, int chunk) {
  return *reinterpret_cast<const u32x4_t*>(t + tile_off<D>(r, chunk));
}

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Transposed operand of a row-major tile X via two ds_read_b64_tr_b16: lane l gets
// X[r0 + 8*(l/32) + t][c0 + l%32] in slot t = 0..7, i.e. the MFMA operand of X^T for the 16
// rows r0 .. r0+15 and 32 columns c0 .. c0+31 (r0 % 16 == 0, c0 % 32 == 0).
// Each 16-lane group of ds_read_b64_tr_b16 transposes a 4-row x 16-column block: lane j
// addresses row j/4, columns 4*(j%4) .. +3, and lane i receives column i of the block.
template <int D>
__device__ __forceinline__ u32x4_t tile_col8(const uint16_t* t, int r0, int c0, int lane) {
  const int grp = lane >> 4, li = lane & 15;
  const int col = c0 + 16 * (grp & 1) + 4 * (li & 3);
  const int row = r0 + 8 * (grp >> 1) + (li >> 2);
  const int chunk = col >> 3, sub = col & 7;
  const uint16_t* a0 = t + tile_off<D>(row, chunk) + sub;
  const uint16_t* a1 = t + tile_off<D>(row + 4, chunk) + sub;
  const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a0));
  const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a1));
  const u32x2_t w0 = __builtin_bit_cast(u32x2_t, v0);
  const u32x2_t w1 = __builtin_bit_cast(u32x2_t, v1);
  return u32x4_t{w0[0], w0[1], w1[0], w1[1]};
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2). Map hardware
// block ids so that consecutive work items land on the same XCD: XCD x runs items
// [x * n/8, (x+1) * n/8). Bijective on [0, n).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int n8 = n & ~7;
  if (bid >= n8) return bid;
  return (bid & 7) * (n8 >> 3) + (bid >> 3);
}

}  // namespace cpa
