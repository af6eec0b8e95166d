// One ring step of the forward in fp32 on the vector ALUs (no MFMA): one thread per query row,
// keys staged through LDS 32 at a time, online softmax per row. Meant for small cases that need
// fp32 accuracy; the bf16 MFMA kernel is the throughput path.
#include <math.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace cpa {
namespace {

constexpr int kRows = 64;   // query rows (threads) per workgroup
constexpr int kKeys = 32;   // keys per LDS tile

template <int D>
__global__ void __launch_bounds__(kRows) fwd_f32_kernel(StepParams p) {
  __shared__ float sk[kKeys][D];
  __shared__ float sv[kKeys][D];
  const int n_qt = (p.len_q + kRows - 1) / kRows;
  const int qt = blockIdx.x % n_qt;
  const int h = blockIdx.x / n_qt;
  const int g = h / p.group;
  const int i = qt * kRows + threadIdx.x;
  const bool ok = i < p.len_q;
  const float* qrow = static_cast<const float*>(p.q) + ((size_t)h * p.len_q + (ok ? i : 0)) * D;
  const float* kg = static_cast<const float*>(p.k) + (size_t)g * p.len_kv * D;
  const float* vg = static_cast<const float*>(p.v) + (size_t)g * p.len_kv * D;

  float q[D], o[D];
#pragma unroll
  for (int t = 0; t < D; ++t) {
    q[t] = ok ? qrow[t] : 0.f;
    o[t] = 0.f;
  }
  const int last_row = min((qt + 1) * kRows, p.len_q) - 1;
  long long nk = p.len_kv;
  if (p.causal) nk = min(nk, p.q_pos0 + last_row - p.kv_pos0 + 1);
  const long long qpos = p.q_pos0 + i;
  float m = -INFINITY, l = 0.f;

  for (long long k0 = 0; k0 < nk; k0 += kKeys) {
    for (int e = threadIdx.x; e < kKeys * D; e += kRows) {
      const int r = e / D, t = e % D;
      const long long key = k0 + r;
      const bool kin = key < p.len_kv;
      sk[r][t] = kin ? kg[key * D + t] : 0.f;
      sv[r][t] = kin ? vg[key * D + t] : 0.f;
    }
    __syncthreads();
    float s[kKeys];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < kKeys; ++r) {
      const long long key = k0 + r;
      float dot = 0.f;
#pragma unroll
      for (int t = 0; t < D; ++t) dot = fmaf(q[t], sk[r][t], dot);
      const bool vis = key < p.len_kv && (!p.causal || p.kv_pos0 + key <= qpos);
      s[r] = vis ? dot * p.scale : -INFINITY;
      mt = fmaxf(mt, s[r]);
    }
    const float m_new = fmaxf(m, mt);
    if (m_new != -INFINITY) {
      const float corr = expf(m - m_new);
      l *= corr;
#pragma unroll
      for (int t = 0; t < D; ++t) o[t] *= corr;
#pragma unroll
      for (int r = 0; r < kKeys; ++r) {
        const float pr = expf(s[r] - m_new);
        l += pr;
#pragma unroll
        for (int t = 0; t < D; ++t) o[t] = fmaf(pr, sv[r][t], o[t]);
      }
      m = m_new;
    }
    __syncthreads();
  }
  if (!ok) return;
  float* orow = p.o + ((size_t)h * p.len_q + i) * D;
  float* lrow = p.lse + (size_t)h * p.len_q + i;
  const float lse_new = l > 0.f ? m + logf(l) : -INFINITY;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (!p.accumulate) {
#pragma unroll
    for (int t = 0; t < D; ++t) orow[t] = o[t] * inv;
    *lrow = lse_new;
  } else if (lse_new != -INFINITY) {
    const float lse_old = *lrow;
    const float hi = fmaxf(lse_old, lse_new);
    const float lse_m = hi + log1pf(expf(-fabsf(lse_old - lse_new)));
    const float wa = expf(lse_old - lse_m);
    const float wb = expf(lse_new - lse_m) * inv;
#pragma unroll
    for (int t = 0; t < D; ++t) orow[t] = wa * orow[t] + wb * o[t];
    *lrow = lse_m;
  }
}

template <int D>
hipError_t launch_d(const StepParams& p, hipStream_t s) {
  const int n_qt = (p.len_q + kRows - 1) / kRows;
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3((unsigned)(n_qt * p.heads_q)), dim3(kRows), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const StepParams& p, hipStream_t s) {
  if (p.head_dim == 128) return launch_d<128>(p, s);
  if (p.head_dim == 64) return launch_d<64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace cpa
