// Context-parallel causal FIR convolution on gfx950 (StripedHyena 2 context-parallelism page,
// section 3, p2p convolution): the zero-history local stage, the sender's halo pack and the
// boundary (halo) stage.
//
// Local stage. A workgroup of 256 threads produces 2048 consecutive outputs of one channel: it
// stages the samples t0 - TP .. t0 + 2047 (TP = taps rounded up to 8; zeros before the start
// and past the end) in LDS as fp32, and each thread computes 8 consecutive outputs with
// fp32 FMAs, walking the taps in groups of 8 with a 16-sample register window that slides back
// by 8 samples per group (two 16-byte LDS reads per 64 FMAs). The filter is read from LDS as
// broadcast reads. With few taps the stage is bound by HBM (2 or 4 bytes read and 4 written
// per output); with many it would be bound by the VALU (2 * taps flops per output).
//
// Local stage on the matrix cores (bf16, 16 < taps <= 256). Cut the outputs of one channel into
// blocks of 32 samples, y[32m + i], and the inputs likewise, X[j][m] = x[32m + j]. Then
//     y[32m + i] = sum_b sum_j h[i - j + 32b] * X[j][m - b],   b = 0 .. bmax,
// with h taken as zero outside [0, taps): a Toeplitz matrix [32 x 32(bmax + 1)] built once per
// channel from h times the matrix of shifted input blocks, i.e. a bf16 MFMA product with fp32
// accumulation whose A operand stays in registers. One wavefront produces 32 blocks (1024
// outputs) with 2(bmax + 1) MFMAs, reading its B operands from the bf16 input tile in LDS.
// The products are exact (bf16 x bf16 in fp32); only the fp32 summation order differs from the
// VALU form. 25% more multiply-adds than the direct form, at matrix-core rates: the stage
// becomes bound by HBM again.
#include "device_common.hpp"
#include "kernels.hpp"

namespace cpa {
namespace {

// Output rows are written once and not read again by these kernels: streaming stores (1) or
// plain stores (0).
#ifndef CP_FIR_NT_STORE
#define CP_FIR_NT_STORE 1
#endif
__device__ __forceinline__ void store4(float* dst, f32x4_t v) {
  if constexpr (CP_FIR_NT_STORE)
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(dst));
  else
    *reinterpret_cast<f32x4_t*>(dst) = v;
}

constexpr int kThreads = 256;
constexpr int kPer = 8;                 // outputs per thread
constexpr int kTile = kThreads * kPer;  // outputs per workgroup
constexpr int kMaxTaps = 1024;

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) {
  return __uint_as_float((uint32_t)v << 16);
}

// Eight consecutive samples starting at element t of row x (t a multiple of 8, all in range),
// as fp32.
template <typename T>
__device__ __forceinline__ void load8(const T* x, long long t, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(x + t);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_lo(w[e]);
      v[2 * e + 1] = bf16_hi(w[e]);
    }
  } else {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(x + t);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(x + t + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  }
}

// VEC: rows are a multiple of 8 samples long, so every group of 8 is 16-byte aligned.
template <typename T, bool VEC>
__global__ void __launch_bounds__(kThreads) fir_local_kernel(FirParams p) {
  __shared__ __attribute__((aligned(16))) float xs[kTile + kMaxTaps];
  __shared__ __attribute__((aligned(16))) float hs[kMaxTaps];
  const int tid = threadIdx.x;
  const int n_tiles = (p.len + kTile - 1) / kTile;
  const long long b = blockIdx.x;
  const int tile = (int)(b % n_tiles);
  const long long row = b / n_tiles;              // shard * channels + channel
  const int c = (int)(row % p.channels);
  const int TP = p.taps_pad;
  const T* x = static_cast<const T*>(p.x) + row * p.len;
  const T* h = static_cast<const T*>(p.h) + (long long)c * p.taps;
  float* y = p.y + row * p.len;
  const int t0 = tile * kTile;

  for (int k = tid; k < TP; k += kThreads) hs[k] = k < p.taps ? to_f32(h[k]) : 0.f;
  // xs[s] = x[t0 - TP + s], s in [0, TP + kTile), zero outside [0, len)
  for (int s = 8 * tid; s < TP + kTile; s += 8 * kThreads) {
    const int t = t0 - TP + s;
    float v[8];
    if (VEC && t >= 0 && t + 8 <= p.len) {
      load8<T>(x, t, v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (t + e >= 0 && t + e < p.len) ? to_f32(x[t + e]) : 0.f;
    }
    *reinterpret_cast<f32x4_t*>(xs + s) = f32x4_t{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4_t*>(xs + s + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
  }
  __syncthreads();

  // Output j0 + i (i < 8) with tap k reads sample j0 + i - k, at xs[TP + j0 + i - k]. For the
  // taps k0 .. k0 + 7 the window win[m] = xs[TP + j0 - k0 - 8 + m], m < 16, covers them all.
  const int j0 = kPer * tid;
  float acc[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) acc[i] = 0.f;
  float win[16];
  {
    const float* w = xs + TP + j0 - 8;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(w + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) win[4 * q + e] = v[e];
    }
  }
  for (int k0 = 0; k0 < TP; k0 += 8) {
    const f32x4_t ha = *reinterpret_cast<const f32x4_t*>(hs + k0);
    const f32x4_t hb = *reinterpret_cast<const f32x4_t*>(hs + k0 + 4);
    const float hk[8] = {ha[0], ha[1], ha[2], ha[3], hb[0], hb[1], hb[2], hb[3]};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int i = 0; i < kPer; ++i) acc[i] = __builtin_fmaf(hk[kk], win[8 + i - kk], acc[i]);
    if (k0 + 8 < TP) {
      // next group of taps: the window moves 8 samples earlier
#pragma unroll
      for (int m = 0; m < 8; ++m) win[8 + m] = win[m];
      const float* w = xs + TP + j0 - k0 - 16;
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(w);
      const f32x4_t bq = *reinterpret_cast<const f32x4_t*>(w + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        win[e] = a[e];
        win[4 + e] = bq[e];
      }
    }
  }

  const int t = t0 + j0;
  if (VEC && t + 8 <= p.len) {
    store4(y + t, f32x4_t{acc[0], acc[1], acc[2], acc[3]});
    store4(y + t + 4, f32x4_t{acc[4], acc[5], acc[6], acc[7]});
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (t + i < p.len) y[t + i] = acc[i];
  }
}

// halo[row, j] = x[row, len - (taps - 1) + j]: one thread per halo sample.
template <typename T>
__global__ void __launch_bounds__(256) fir_pack_kernel(FirParams p, long long total) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int hl = p.taps - 1;
  const long long row = i / hl;
  const int j = (int)(i % hl);
  static_cast<T*>(p.halo)[i] = static_cast<const T*>(p.x)[row * p.len + p.len - hl + j];
}

// Boundary stage: one wavefront per target row: y[i] += sum_{k > i} h[k] halo[taps-1+i-k],
// i < taps - 1, with the row's filter and halo staged in LDS first (coalesced loads); four
// independent partial sums per output keep the LDS reads in flight. Target row y_row0 + b
// reads halo row b; a workgroup takes kHaloRows consecutive rows.
constexpr int kHaloRows = 4;

template <typename T>
__global__ void __launch_bounds__(64 * kHaloRows) fir_halo_kernel(FirParams p, long long y_row0,
                                                                  long long rows) {
  __shared__ float hs[kHaloRows][kMaxTaps];
  __shared__ float tl[kHaloRows][kMaxTaps];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long b = (long long)blockIdx.x * kHaloRows + wave;
  if (b >= rows) return;  // whole wavefronts only; no workgroup barrier follows
  const int c = (int)((y_row0 + b) % p.channels);
  const int hl = p.taps - 1;
  const T* halo = static_cast<const T*>(p.halo) + b * hl;
  const T* h = static_cast<const T*>(p.h) + (long long)c * p.taps;
  float* y = p.y + (y_row0 + b) * p.len;
  float* hw = hs[wave];
  float* tw = tl[wave];
  for (int k = lane; k < p.taps; k += 64) hw[k] = to_f32(h[k]);
  for (int j = lane; j < hl; j += 64) tw[j] = to_f32(halo[j]);
  __builtin_amdgcn_wave_barrier();  // a wavefront's LDS accesses complete in order
  for (int i = lane; i < hl; i += 64) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    int k = i + 1;
    for (; k + 3 < p.taps; k += 4) {
      a0 = __builtin_fmaf(hw[k], tw[hl + i - k], a0);
      a1 = __builtin_fmaf(hw[k + 1], tw[hl + i - k - 1], a1);
      a2 = __builtin_fmaf(hw[k + 2], tw[hl + i - k - 2], a2);
      a3 = __builtin_fmaf(hw[k + 3], tw[hl + i - k - 3], a3);
    }
    for (; k < p.taps; ++k) a0 = __builtin_fmaf(hw[k], tw[hl + i - k], a0);
    y[i] += (a0 + a1) + (a2 + a3);
  }
}

constexpr int kMfmaMaxTaps = 256;
constexpr int kMfmaWaves = 4;
constexpr int kMfmaTile = kMfmaWaves * 1024;      // outputs per workgroup

// LDS chunk (8 bf16 samples) c is stored at chunk c ^ ((c >> 4) & 3), so that the 32 lanes of
// a B-operand read (chunks 4m + const, m = 0 .. 31) hit distinct banks.
__device__ __forceinline__ int fir_chunk_swz(int c) { return c ^ ((c >> 4) & 3); }

// BMAX: input blocks back that the longest tap reaches, (taps + 30) / 32 (compile-time, so the
// A operands take 8 (BMAX + 1) registers and no more).
template <int BMAX>
__global__ void __launch_bounds__(64 * kMfmaWaves) fir_local_mfma_kernel(FirParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[32 * BMAX + kMfmaTile];
  __shared__ float hz[kMfmaMaxTaps + 64];     // h[k] at hz[k + 32], zero around it
  __shared__ __attribute__((aligned(16))) float os[1024 * kMfmaWaves];  // per-wave output
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, col = lane & 31, half = lane >> 5;
  const int n_tiles = (p.len + kMfmaTile - 1) / kMfmaTile;
  const long long row = blockIdx.x;             // one workgroup per row, tiles in sequence
  const int c = (int)(row % p.channels);
  constexpr int pad = 32 * BMAX;                // history samples this channel needs
  constexpr int nk = 2 * (BMAX + 1);            // K-blocks of 16
  const uint16_t* x = static_cast<const uint16_t*>(p.x) + row * p.len;
  const uint16_t* h = static_cast<const uint16_t*>(p.h) + (long long)c * p.taps;
  float* y = p.y + row * p.len;

  for (int k = tid; k < kMfmaMaxTaps + 64; k += 64 * kMfmaWaves) {
    const int tap = k - 32;
    hz[k] = (tap >= 0 && tap < p.taps) ? bf16_lo((uint32_t)h[tap]) : 0.f;
  }
  __syncthreads();

  // A operand of K-block kk (b = kk / 2, j = 16 (kk % 2) + 8 half + t): h[i - j + 32 b], i = col.
  u32x4_t a[nk];
#pragma unroll
  for (int kk = 0; kk < nk; ++kk) {
    const int base = col - 16 * (kk & 1) - 8 * half + 32 * (kk >> 1) + 32;  // + 32: hz offset
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(hz[base - 2 * e], hz[base - 2 * e - 1]);
    a[kk] = u32x4_t{w[0], w[1], w[2], w[3]};
  }

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int t0 = tile * kMfmaTile;
    if (tile > 0) __syncthreads();  // every wave is done with the previous tile
    // xs chunk q (samples 8q .. 8q+7 of the staged range) = x[t0 - pad + 8q ...], zero outside
    const int n_chunks = (pad + kMfmaTile) / 8;
    for (int q = tid; q < n_chunks; q += 64 * kMfmaWaves) {
      const int t = t0 - pad + 8 * q;
      u32x4_t v;
      if (t >= 0 && t + 8 <= p.len && p.len % 8 == 0) {
        v = *reinterpret_cast<const u32x4_t*>(x + t);
      } else {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ta = t + 2 * e, tb = t + 2 * e + 1;
          const uint32_t lo = (ta >= 0 && ta < p.len) ? x[ta] : 0u;
          const uint32_t hi = (tb >= 0 && tb < p.len) ? x[tb] : 0u;
          w[e] = lo | (hi << 16);
        }
        v = u32x4_t{w[0], w[1], w[2], w[3]};
      }
      *reinterpret_cast<u32x4_t*>(xs + 8 * fir_chunk_swz(q)) = v;
    }

    __syncthreads();
    // This wave's 1024 outputs: t0 + 1024 wave + 32 m + i.
    const int w0 = 1024 * wave;
    if (t0 + w0 >= p.len) continue;
    f32x16_t acc = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < nk; ++kk) {
      // B operand: x[t0 + w0 + 32 (col - b) + 16 (kk % 2) + 8 half + t], t = 0..7
      const int sidx = pad + w0 + 32 * (col - (kk >> 1)) + 16 * (kk & 1) + 8 * half;
      const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(xs + 8 * fir_chunk_swz(sidx >> 3));
      acc = mfma32x32x16(a[kk], bv, acc);
    }
    // acc register r: row i = 8 (r / 4) + 4 half + r % 4 of output block m = col. Reorder the
    // wave's 1024 outputs through LDS so that the stores are contiguous 16-byte runs.
    float* ow = os + 1024 * wave;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<f32x4_t*>(ow + 32 * col + 8 * g + 4 * half) =
          f32x4_t{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    // a wavefront's LDS accesses complete in order: its reads below see these writes
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int o = 256 * q + 4 * lane;
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(ow + o);
      const int t = t0 + w0 + o;
      if (t + 4 <= p.len && p.len % 4 == 0) {
        store4(y + t, v);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (t + e < p.len) y[t + e] = v[e];
      }
    }
  }
}

template <typename T>
hipError_t launch_local_t(const FirParams& p, long long rows, hipStream_t s) {
  const long long n_tiles = (p.len + kTile - 1) / kTile;
  const dim3 grid((unsigned)(n_tiles * rows));
  if (p.len % 8 == 0)
    hipLaunchKernelGGL((fir_local_kernel<T, true>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((fir_local_kernel<T, false>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fir_local(const FirParams& p, long long rows, hipStream_t s) {
  if (rows <= 0 || p.len <= 0) return hipSuccess;
  if (p.is_bf16 && p.taps > 16 && p.taps <= kMfmaMaxTaps) {
    const dim3 grid((unsigned)rows), block(64 * kMfmaWaves);
    switch ((p.taps + 30) / 32) {
      case 1: hipLaunchKernelGGL(fir_local_mfma_kernel<1>, grid, block, 0, s, p); break;
      case 2: hipLaunchKernelGGL(fir_local_mfma_kernel<2>, grid, block, 0, s, p); break;
      case 3: hipLaunchKernelGGL(fir_local_mfma_kernel<3>, grid, block, 0, s, p); break;
      case 4: hipLaunchKernelGGL(fir_local_mfma_kernel<4>, grid, block, 0, s, p); break;
      case 5: hipLaunchKernelGGL(fir_local_mfma_kernel<5>, grid, block, 0, s, p); break;
      case 6: hipLaunchKernelGGL(fir_local_mfma_kernel<6>, grid, block, 0, s, p); break;
      case 7: hipLaunchKernelGGL(fir_local_mfma_kernel<7>, grid, block, 0, s, p); break;
      default: hipLaunchKernelGGL(fir_local_mfma_kernel<8>, grid, block, 0, s, p); break;
    }
    return hipGetLastError();
  }
  return p.is_bf16 ? launch_local_t<uint16_t>(p, rows, s) : launch_local_t<float>(p, rows, s);
}

hipError_t launch_fir_pack(const FirParams& p, long long rows, hipStream_t s) {
  const long long total = rows * (p.taps - 1);
  if (total <= 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (p.is_bf16)
    hipLaunchKernelGGL((fir_pack_kernel<uint16_t>), grid, dim3(256), 0, s, p, total);
  else
    hipLaunchKernelGGL((fir_pack_kernel<float>), grid, dim3(256), 0, s, p, total);
  return hipGetLastError();
}

hipError_t launch_fir_halo(const FirParams& p, long long y_row0, long long rows, hipStream_t s) {
  if (rows <= 0 || p.taps <= 1) return hipSuccess;
  const dim3 grid((unsigned)((rows + kHaloRows - 1) / kHaloRows));
  if (p.is_bf16)
    hipLaunchKernelGGL((fir_halo_kernel<uint16_t>), grid, dim3(64 * kHaloRows), 0, s, p, y_row0,
                       rows);
  else
    hipLaunchKernelGGL((fir_halo_kernel<float>), grid, dim3(64 * kHaloRows), 0, s, p, y_row0,
                       rows);
  return hipGetLastError();
}

}  // namespace cpa
