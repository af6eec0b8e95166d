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

// Row-major bf16 tile of D columns in LDS (64 banks of 4 bytes: a ds_read_b128 serves 16 lanes
// per pass, a ds_read_b64 32 lanes). Its 16-byte chunks are XOR-swizzled per row:
//  * bits 2-3 of the swizzle = row % 4, so the 4 consecutive rows a transpose read touches land
//    in 4 different 64-byte quarters of the 256-byte bank window;
//  * bits 0-1 = rows bits 3 and 2, so the 16 rows perm_row(0..15) of a row read land on 16
//    different chunk positions.
// (For d = 64 a row is half the bank window, so row bit 1 takes the place of row % 4.)
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  if constexpr (D >= 128) return ((r & 3) << 2) | ((r >> 3) & 1) | (((r >> 2) & 1) << 1);
  else return (((r >> 1) & 1) << 2) | ((r >> 3) & 1) | (((r >> 2) & 1) << 1);
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

// Buffer resource over `bytes` bytes at `base`: loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// LDS byte offset of a pointer into LDS: the low 32 bits of its generic address (the LDS
// aperture sits above 4 GB). Cheaper than the address-space cast, which tests for null.
__device__ __forceinline__ unsigned lds_offset(const void* p) {
  return (unsigned)(uintptr_t)p;
}

// One direct global -> LDS load: 16 bytes per lane from `rsrc` at byte offset `voff` into the
// LDS block starting at byte offset `lds_off` (wave-uniform; lane i's bytes land at
// lds_off + 16 i). Issued as an explicit instruction rather than through the compiler's
// builtin, which makes every later LDS read that the compiler cannot prove disjoint from the
// destination wait for the load (vmcnt), and would so serialise a double-buffered pipeline on
// its own prefetch. The caller is responsible for completion: s_waitcnt vmcnt(0) and a
// workgroup barrier before anything reads the block.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, unsigned voff,
                                          unsigned lds_off) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(lds_off)
               : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding (LDS and export
// counters untouched). Vector loads complete in issue order, so this waits for all but the N
// most recent ones. s_waitcnt encoding of the gfx9 family: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4 (7 = no wait), lgkmcnt in 11:8 (15 = no wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Direct global -> LDS copy of a ROWS x D bf16 tile into the swizzled layout (no registers, no
// LDS store instructions). One buffer_load_dwordx4 ... lds per wave fills 1 KB of LDS at
// consecutive 16-byte slots, i.e. 1024 / (2D) whole rows; each lane fetches the source chunk that
// belongs at its slot. The tile's first row goes into the buffer descriptor's base (scalar
// arithmetic), so the per-lane offsets stay loop-invariant; rows at or past `nrows` read as
// zeros. Completion is tracked by vmcnt: wait for it before the barrier that publishes the tile.
// `wave` is the caller's wavefront index (the same in every lane).
template <int D, int ROWS, int NT>
struct TileDma {
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int RPI = 64 / CH;              // rows per wave instruction
  static constexpr int NWAVE = NT / 64;
  static constexpr int ITERS = ROWS / (RPI * NWAVE);
  static_assert(ROWS % (RPI * NWAVE) == 0, "tile must split evenly over the waves");
  // LDS byte offset of this wave's first block of the tile; the wave's later blocks follow at
  // a fixed stride.
  __device__ __forceinline__ static unsigned wave_base(const uint16_t* lds_tile, int wave) {
    return __builtin_amdgcn_readfirstlane(lds_offset(lds_tile + wave * RPI * D));
  }
  static constexpr unsigned kStride = NWAVE * RPI * D * 2;  // bytes between a wave's blocks

  __device__ __forceinline__ static void issue(const uint16_t* src, int row0, int nrows,
                                               uint16_t* lds_tile, int wave, int lane) {
    const __amdgpu_buffer_rsrc_t rsrc =
        make_rsrc(src + (size_t)row0 * D, (unsigned)(nrows - row0) * D * 2u);
    const unsigned base = wave_base(lds_tile, wave);
#pragma unroll
    for (int u = 0; u < ITERS; ++u) {
      const int r = (u * NWAVE + wave) * RPI + lane / CH;
      const int c = (lane % CH) ^ tile_swz<D>(r);
      const unsigned voff = ((unsigned)r * D + 8u * c) * 2u;
      lds_dma16(rsrc, voff, base + u * kStride);
    }
  }
  // Same copy with the tile's row offset folded into each lane's offset instead of the
  // descriptor: a few more vector instructions per tile, but no offsets kept live across a loop
  // (for kernels at the edge of their register budget).
  __device__ __forceinline__ static void issue_lean(const uint16_t* src, int row0, int nrows,
                                                    uint16_t* lds_tile, int wave, int lane) {
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(src, (unsigned)nrows * D * 2u);
    const unsigned base = wave_base(lds_tile, wave);
#pragma unroll
    for (int u = 0; u < ITERS; ++u) {
      const int r = (u * NWAVE + wave) * RPI + lane / CH;
      const int c = (lane % CH) ^ tile_swz<D>(r);
      const unsigned voff = ((unsigned)(row0 + r) * D + 8u * c) * 2u;
      lds_dma16(rsrc, voff, base + u * kStride);
    }
  }
};

// N matrix products step(i, A_i) whose A operands are LDS reads load(i), each read issued PF
// products ahead of its use; scheduling fences keep that order (the compiler would otherwise
// pull reads next to their product and expose the LDS latency).
template <int N, int PF, typename LA, typename ST>
__device__ __forceinline__ void mfma_seq(LA load, ST step) {
  u32x4_t ra[N];
#pragma unroll
  for (int i = 0; i < PF && i < N; ++i) ra[i] = load(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + PF < N) ra[i + PF] = load(i + PF);
    step(i, ra[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Causal visibility in chunk-local coordinates: key j is visible to query i iff
// kv_pos0 + j <= q_pos0 + i, i.e. j - i <= q_pos0 - kv_pos0. The difference is clamped to a
// range where the 32-bit test stays exact for local indices below 2^24.
__device__ __forceinline__ int causal_shift(long long q_pos0, long long kv_pos0) {
  const long long d = q_pos0 - kv_pos0;
  return (int)(d > (1ll << 30) ? (1ll << 30) : (d < -(1ll << 30) ? -(1ll << 30) : d));
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
