// Parameter blocks and launchers of the gfx950 kernels (internal to the library; the public
// boundary is include/cp_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpa {

struct StepParams {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  int heads_q, heads_kv, group;
  int len_q, len_kv, head_dim;
  long long q_pos0, kv_pos0;
  int causal;
  int accumulate;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* d_o;
  const float* lse;
  const float* delta;
  float* dq;
  float* dk;
  float* dv;
  int heads_q, heads_kv, group;
  int len_q, len_kv, head_dim;
  long long q_pos0, kv_pos0;
  int causal;
  float scale;
  float scale_log2;
};

// Compute units of the current device (queried once per device).
int device_cus();

hipError_t launch_fwd_bf16(const StepParams& p, hipStream_t s);
hipError_t launch_fwd_f32(const StepParams& p, hipStream_t s);
hipError_t launch_merge(long long rows, int head_dim, float* o_acc, float* lse_acc,
                        const float* o, const float* lse, hipStream_t s);
hipError_t launch_bwd_prep(long long rows, int head_dim, int is_bf16, const float* o,
                           const void* d_o, float* delta, hipStream_t s);
// which: 1 = dK/dV kernel, 2 = dQ kernel, 3 = both.
hipError_t launch_bwd_bf16(const BwdParams& p, int which, hipStream_t s);

// Causal FIR convolution. Rows are (shard, channel) pairs of `len` samples; x, y, halo are
// indexed by row, h by channel (row % channels).
struct FirParams {
  const void* x;     // [rows, len] (dtype)
  const void* h;     // [channels, taps] (dtype)
  void* halo;        // [rows, taps - 1] (dtype)
  float* y;          // [rows, len] fp32
  int channels, len, taps, taps_pad;  // taps_pad: taps rounded up to a multiple of 8
  int is_bf16;
};
hipError_t launch_fir_local(const FirParams& p, long long rows, hipStream_t s);
hipError_t launch_fir_pack(const FirParams& p, long long rows, hipStream_t s);
// y rows y_row0 .. y_row0 + rows - 1 take the boundary terms of halo rows 0 .. rows - 1.
hipError_t launch_fir_halo(const FirParams& p, long long y_row0, long long rows, hipStream_t s);

}  // namespace cpa
