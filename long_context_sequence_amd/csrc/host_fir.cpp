// Host side of the C ABI declared in include/cp_fir.h: validation and kernel dispatch for the
// context-parallel causal FIR convolution. Nothing is allocated here.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "cp_fir.h"
#include "kernels.hpp"

namespace {

constexpr int64_t kTileOutputs = 2048;  // outputs per workgroup of the local stage

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

cp_status from_hip(hipError_t e) { return e == hipSuccess ? CP_OK : CP_ERR_HIP; }

cp_status check(const cp_fir_desc* d, int64_t shards) {
  if (!d) return CP_ERR_NULL;
  if (d->channels < 1 || d->channels > CP_FIR_MAX_CHANNELS) return CP_ERR_SHAPE;
  if (d->shard_len < 0 || d->shard_len > CP_MAX_LEN) return CP_ERR_SHAPE;
  if (d->taps < 1 || d->taps > CP_FIR_MAX_TAPS || d->taps - 1 > d->shard_len) return CP_ERR_SHAPE;
  if (d->dtype != CP_F32 && d->dtype != CP_BF16) return CP_ERR_DTYPE;
  const int64_t rows = shards * d->channels;
  const int64_t tiles = (d->shard_len + kTileOutputs - 1) / kTileOutputs;
  if (rows * tiles >= ((int64_t)1 << 31)) return CP_ERR_SHAPE;  // one launch's grid
  return CP_OK;
}

cp_status check_ptrs(const void* a, const void* b, const void* c) {
  for (const void* p : {a, b, c})
    if (!p) return CP_ERR_NULL;
  for (const void* p : {a, b, c})
    if (!aligned16(p)) return CP_ERR_ALIGN;
  return CP_OK;
}

cpa::FirParams params(const cp_fir_desc* d, const void* x, const void* h, void* halo, float* y) {
  cpa::FirParams p;
  p.x = x;
  p.h = h;
  p.halo = halo;
  p.y = y;
  p.channels = d->channels;
  p.len = d->shard_len;
  p.taps = d->taps;
  p.taps_pad = (d->taps + 7) / 8 * 8;
  p.is_bf16 = d->dtype == CP_BF16;
  return p;
}

}  // namespace

extern "C" {

cp_status cp_fir_local(const cp_fir_desc* desc, const void* x, const void* h, float* y,
                       void* stream) {
  cp_status st = check(desc, 1);
  if (st != CP_OK) return st;
  if (desc->shard_len == 0) return CP_OK;
  st = check_ptrs(x, h, y);
  if (st != CP_OK) return st;
  return from_hip(cpa::launch_fir_local(params(desc, x, h, nullptr, y), desc->channels,
                                        static_cast<hipStream_t>(stream)));
}

cp_status cp_fir_pack_halo(const cp_fir_desc* desc, const void* x, void* halo, void* stream) {
  cp_status st = check(desc, 1);
  if (st != CP_OK) return st;
  if (desc->taps == 1) return CP_OK;
  st = check_ptrs(x, halo, x);
  if (st != CP_OK) return st;
  return from_hip(cpa::launch_fir_pack(params(desc, x, nullptr, halo, nullptr), desc->channels,
                                       static_cast<hipStream_t>(stream)));
}

cp_status cp_fir_halo(const cp_fir_desc* desc, const void* halo, const void* h, float* y,
                      void* stream) {
  cp_status st = check(desc, 1);
  if (st != CP_OK) return st;
  if (desc->taps == 1) return CP_OK;
  st = check_ptrs(halo, h, y);
  if (st != CP_OK) return st;
  return from_hip(cpa::launch_fir_halo(params(desc, nullptr, h, const_cast<void*>(halo), y), 0,
                                       desc->channels, static_cast<hipStream_t>(stream)));
}

cp_status cp_fir_ring(const cp_fir_desc* desc, int32_t n_cp, const void* x_shards,
                      const void* h, void* halo_work, float* y_shards, void* stream) {
  if (n_cp < 1 || n_cp > (1 << 16)) return desc ? CP_ERR_SHAPE : CP_ERR_NULL;
  cp_status st = check(desc, n_cp);
  if (st != CP_OK) return st;
  if (desc->shard_len == 0) return CP_OK;
  st = check_ptrs(x_shards, h, y_shards);
  if (st != CP_OK) return st;
  const bool halo = desc->taps > 1 && n_cp > 1;
  if (halo) {
    if (!halo_work) return CP_ERR_NULL;
    if (!aligned16(halo_work)) return CP_ERR_ALIGN;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t rows = (int64_t)n_cp * desc->channels;
  const cpa::FirParams p = params(desc, x_shards, h, halo_work, y_shards);
  // the senders' side: every shard's tail (the last shard's is never used)
  if (halo) {
    st = from_hip(cpa::launch_fir_pack(p, rows - desc->channels, s));
    if (st != CP_OK) return st;
  }
  // stage one on every shard; on a ring of GPUs this overlaps the halo exchange
  st = from_hip(cpa::launch_fir_local(p, rows, s));
  if (st != CP_OK) return st;
  // stage two: shard r (r >= 1) takes shard r - 1's tail
  if (halo) st = from_hip(cpa::launch_fir_halo(p, desc->channels, rows - desc->channels, s));
  return st;
}

}  // extern "C"
