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
// per output); with many it is bound by the VALU (2 * taps flops per output).
#include "device_common.hpp"
#include "kernels.hpp"

namespace cpa {
namespace {

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
    *reinterpret_cast<f32x4_t*>(y + t) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4_t*>(y + t + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
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
// i < taps - 1, with the row's filter and halo staged in LDS first (coalesced loads).
// Target row y_row0 + b reads halo row b.
template <typename T>
__global__ void __launch_bounds__(64) fir_halo_kernel(FirParams p, long long y_row0) {
  __shared__ float hs[kMaxTaps];
  __shared__ float tl[kMaxTaps];
  const long long b = blockIdx.x;
  const int c = (int)((y_row0 + b) % p.channels);
  const int hl = p.taps - 1;
  const T* halo = static_cast<const T*>(p.halo) + b * hl;
  const T* h = static_cast<const T*>(p.h) + (long long)c * p.taps;
  float* y = p.y + (y_row0 + b) * p.len;
  for (int k = threadIdx.x; k < p.taps; k += 64) hs[k] = to_f32(h[k]);
  for (int j = threadIdx.x; j < hl; j += 64) tl[j] = to_f32(halo[j]);
  __syncthreads();
  for (int i = threadIdx.x; i < hl; i += 64) {
    float acc = 0.f;
    for (int k = i + 1; k < p.taps; ++k) acc = __builtin_fmaf(hs[k], tl[hl + i - k], acc);
    y[i] += acc;
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
  const dim3 grid((unsigned)rows);
  if (p.is_bf16)
    hipLaunchKernelGGL((fir_halo_kernel<uint16_t>), grid, dim3(64), 0, s, p, y_row0);
  else
    hipLaunchKernelGGL((fir_halo_kernel<float>), grid, dim3(64), 0, s, p, y_row0);
  return hipGetLastError();
}

}  // namespace cpa
