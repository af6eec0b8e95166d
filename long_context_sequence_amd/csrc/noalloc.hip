// The rank's backward ring without a caller-provided workspace: for callers that cannot
// allocate device memory (code under graph capture, serving loops, harnesses that forbid
// allocation). The per-row delta that cp_attn_ring_bwd keeps in `delta_work` lives here in a
// fixed device array instead; everything else is cp_attn_ring_bwd unchanged.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "cp_attn.h"

namespace {

constexpr int64_t kScratchFloats = CP_NOALLOC_MAX_ROWS;  // 16 MiB of fp32
constexpr int kMaxDevices = 64;

// One copy per device, held until the process ends. Host code uses only the device address
// returned by hipGetSymbolAddress (the array's name is a host-side stand-in).
__device__ __align__(256) float scratch[kScratchFloats];

std::mutex g_init_mutex;
float* g_scratch[kMaxDevices] = {nullptr};

// Device address of the current device's array, looked up once per device.
cp_status scratch_address(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CP_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_init_mutex);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return CP_ERR_HIP;
    g_scratch[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch[dev];
  return CP_OK;
}

}  // namespace

extern "C" cp_status cp_attn_ring_bwd_noalloc(const cp_ring_desc* ring, const void* q,
                                              const void* k_chunks, const void* v_chunks,
                                              const void* d_o, const float* o, const float* lse,
                                              float* dq, float* dk_chunks, float* dv_chunks,
                                              void* stream) {
  if (!ring) return CP_ERR_NULL;
  if (ring->heads_q < 1 || ring->chunk_len < 1) return CP_ERR_SHAPE;
  if ((int64_t)ring->heads_q * ring->chunk_len > kScratchFloats) return CP_ERR_SCRATCH_LIMIT;
  float* delta = nullptr;
  const cp_status st = scratch_address(&delta);
  if (st != CP_OK) return st;
  return cp_attn_ring_bwd(ring, q, k_chunks, v_chunks, d_o, o, lse, delta, dq, dk_chunks,
                          dv_chunks, stream);
}
