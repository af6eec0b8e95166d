// HBM-bound passes over the fp32 output rows:
//  * merge: fold one ring step's (O, LSE) into the running (O, LSE) in place (StripedHyena 2
//    context-parallelism page, section 2, ring attention step 3: statistics are updated online);
//  * bwd_prep: delta = rowsum(dO * O), the softmax-Jacobian term of the backward.
// One float4 of O per thread; the head_dim/4 threads of a row sit in one wavefront, so a row's
// LSE is read by all of them before one of them rewrites it.
#include <math.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace cpa {
namespace {

template <int D>
__global__ void __launch_bounds__(256) merge_kernel(long long rows, float* __restrict__ o_acc,
                                                    float* __restrict__ lse_acc,
                                                    const float* __restrict__ o,
                                                    const float* __restrict__ lse) {
  constexpr int V = D / 4;  // float4 per row
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = idx / V;
  if (row >= rows) return;
  const float a = lse_acc[row];
  const float b = __builtin_nontemporal_load(&lse[row]);
  const float hi = fmaxf(a, b);
  float wa = 0.f, wb = 0.f, lnew = -INFINITY;
  if (hi != -INFINITY) {
    lnew = hi + log1pf(expf(-fabsf(a - b)));
    wa = expf(a - lnew);
    wb = expf(b - lnew);
  }
  f32x4_t* pa = reinterpret_cast<f32x4_t*>(o_acc) + idx;
  const f32x4_t x = *pa;
  const f32x4_t y = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(o) + idx);
  f32x4_t r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = wa * x[e] + wb * y[e];
  *pa = r;
  if ((idx % V) == 0) lse_acc[row] = lnew;
}

template <int D, bool BF16>
__global__ void __launch_bounds__(256) prep_kernel(long long rows, const float* __restrict__ o,
                                                   const void* __restrict__ d_o,
                                                   float* __restrict__ delta) {
  // 8 elements per thread (two 16-byte loads of O, one of bf16 dO), D/8 threads per row
  constexpr int V = D / 8;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = idx / V;
  const bool ok = row < rows;
  float acc = 0.f;
  if (ok) {
    const f32x4_t* op = reinterpret_cast<const f32x4_t*>(o) + 2 * idx;
    const f32x4_t x0 = __builtin_nontemporal_load(op);
    const f32x4_t x1 = __builtin_nontemporal_load(op + 1);
    float g[8];
    if constexpr (BF16) {
      const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(d_o) + idx);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        g[2 * t] = bf16_lo(w[t]);
        g[2 * t + 1] = bf16_hi(w[t]);
      }
    } else {
      const f32x4_t* yp = reinterpret_cast<const f32x4_t*>(d_o) + 2 * idx;
      const f32x4_t y0 = __builtin_nontemporal_load(yp);
      const f32x4_t y1 = __builtin_nontemporal_load(yp + 1);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        g[t] = y0[t];
        g[4 + t] = y1[t];
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) acc += x0[t] * g[t] + x1[t] * g[4 + t];
  }
#pragma unroll
  for (int off = V / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, V);
  if (ok && (idx % V) == 0) delta[row] = acc;
}

template <int D>
hipError_t merge_d(long long rows, float* o_acc, float* lse_acc, const float* o, const float* lse,
                   hipStream_t s) {
  const long long threads = rows * (D / 4);
  const long long blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((merge_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, s, rows, o_acc,
                     lse_acc, o, lse);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t prep_d(long long rows, const float* o, const void* d_o, float* delta, hipStream_t s) {
  const long long threads = rows * (D / 8);
  const long long blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((prep_kernel<D, BF16>), dim3((unsigned)blocks), dim3(256), 0, s, rows, o,
                     d_o, delta);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(long long rows, int head_dim, float* o_acc, float* lse_acc,
                        const float* o, const float* lse, hipStream_t s) {
  if (head_dim == 128) return merge_d<128>(rows, o_acc, lse_acc, o, lse, s);
  if (head_dim == 64) return merge_d<64>(rows, o_acc, lse_acc, o, lse, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_prep(long long rows, int head_dim, int is_bf16, const float* o,
                           const void* d_o, float* delta, hipStream_t s) {
  if (head_dim == 128)
    return is_bf16 ? prep_d<128, true>(rows, o, d_o, delta, s) : prep_d<128, false>(rows, o, d_o, delta, s);
  if (head_dim == 64)
    return is_bf16 ? prep_d<64, true>(rows, o, d_o, delta, s) : prep_d<64, false>(rows, o, d_o, delta, s);
  return hipErrorInvalidValue;
}

}  // namespace cpa
