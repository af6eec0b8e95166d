// Sustained-rate probes, timed by the caller:
//  * matrix cores: v_mfma_f32_32x32x16_bf16 with register operands and four independent
//    accumulators per wavefront, nothing else in the loop (beside the published 2.5 PFLOP/s);
//  * HBM: a copy with one 16-byte load and one 16-byte store per thread, the access pattern of
//    the library's elementwise kernels (beside the published 8 TB/s).
#include "cp_probe.h"
#include "device_common.hpp"

namespace cpa {
namespace {

constexpr int kProbeThreads = 256;

__global__ void __launch_bounds__(kProbeThreads) probe_mfma_kernel(int iters, float* sink) {
  const int tid = threadIdx.x;
  // Operands: small finite bf16 values that differ per lane (the rate does not depend on them).
  u32x4_t a, b;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    a[t] = pack_bf16x2(0.001f * (tid + t), 0.002f * t);
    b[t] = pack_bf16x2(0.003f * t, -0.001f * (tid & 7));
  }
  f32x16_t c0 = f32x16_t{}, c1 = f32x16_t{}, c2 = f32x16_t{}, c3 = f32x16_t{};
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32x32x16(a, b, c0);
    c1 = mfma32x32x16(a, b, c1);
    c2 = mfma32x32x16(a, b, c2);
    c3 = mfma32x32x16(a, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[(size_t)blockIdx.x * kProbeThreads + tid] = s;
}

__global__ void __launch_bounds__(256) probe_copy_kernel(long long n4, const f32x4_t* __restrict__ src,
                                                         f32x4_t* __restrict__ dst) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) dst[i] = __builtin_nontemporal_load(src + i);
}

}  // namespace
}  // namespace cpa

extern "C" cp_status cp_probe_mfma_bf16(int32_t workgroups, int32_t iters, float* sink,
                                        void* stream) {
  if (sink == nullptr) return CP_ERR_NULL;
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 20))
    return CP_ERR_SHAPE;
  hipLaunchKernelGGL(cpa::probe_mfma_kernel, dim3((unsigned)workgroups), dim3(cpa::kProbeThreads),
                     0, static_cast<hipStream_t>(stream), (int)iters, sink);
  return hipGetLastError() == hipSuccess ? CP_OK : CP_ERR_HIP;
}

extern "C" cp_status cp_probe_copy(int64_t n_float4, const void* src, void* dst, void* stream) {
  if (src == nullptr || dst == nullptr) return CP_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15)
    return CP_ERR_ALIGN;
  if (n_float4 < 1 || n_float4 > (int64_t(1) << 34)) return CP_ERR_SHAPE;
  const long long blocks = (n_float4 + 255) / 256;
  hipLaunchKernelGGL(cpa::probe_copy_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), (long long)n_float4,
                     static_cast<const cpa::f32x4_t*>(src), static_cast<cpa::f32x4_t*>(dst));
  return hipGetLastError() == hipSuccess ? CP_OK : CP_ERR_HIP;
}
