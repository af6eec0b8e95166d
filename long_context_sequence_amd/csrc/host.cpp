// Host side of the C ABI declared in include/cp_attn.h: argument validation, step
// classification, the ring schedule and kernel dispatch. Nothing is allocated here and no state
// outlives a call.
#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include <hip/hip_runtime.h>

#include "cp_attn.h"
#include "kernels.hpp"

namespace {

constexpr int32_t kAbiVersion = 1;
constexpr int32_t kMaxRing = 1 << 16;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

cp_status from_hip(hipError_t e) {
  if (e == hipSuccess) return CP_OK;
  if (e == hipErrorNotSupported) return CP_ERR_UNSUPPORTED;
  return CP_ERR_HIP;
}

// Shape and flag checks common to the step and the backward step.
cp_status check_desc(const cp_attn_desc* d) {
  if (!d) return CP_ERR_NULL;
  if (d->heads_q < 1 || d->heads_kv < 1 || d->heads_q > CP_MAX_HEADS ||
      d->heads_kv > CP_MAX_HEADS || d->heads_q % d->heads_kv != 0)
    return CP_ERR_SHAPE;
  if (d->len_q < 0 || d->len_kv < 0 || d->len_q > CP_MAX_LEN || d->len_kv > CP_MAX_LEN)
    return CP_ERR_SHAPE;
  if (d->head_dim < 1) return CP_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return CP_ERR_UNSUPPORTED;
  if (d->causal != 0 && d->causal != 1) return CP_ERR_SHAPE;
  if (d->accumulate != 0 && d->accumulate != 1) return CP_ERR_SHAPE;
  if (d->dtype != CP_F32 && d->dtype != CP_BF16) return CP_ERR_DTYPE;
  if (isnan(d->scale) || isinf(d->scale)) return CP_ERR_SHAPE;
  const int64_t lim = (int64_t)1 << 60;
  if (d->q_pos0 < -lim || d->q_pos0 > lim || d->kv_pos0 < -lim || d->kv_pos0 > lim)
    return CP_ERR_SHAPE;
  return CP_OK;
}

// Causal and every key after every query: the step has nothing to do.
bool causally_empty(const cp_attn_desc* d) {
  return d->causal && d->kv_pos0 > d->q_pos0 + (int64_t)d->len_q - 1;
}

float resolve_scale(const cp_attn_desc* d) {
  return d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)d->head_dim);
}

cp_status check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (!p) return CP_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return CP_ERR_ALIGN;
  return CP_OK;
}

cp_status check_ring(const cp_ring_desc* r) {
  if (!r) return CP_ERR_NULL;
  if (r->n_cp < 1 || r->n_cp > kMaxRing || r->rank < 0 || r->rank >= r->n_cp) return CP_ERR_SHAPE;
  if (r->chunk_len < 1) return CP_ERR_SHAPE;
  return CP_OK;
}

cp_attn_desc ring_step_desc(const cp_ring_desc* r, int32_t chunk, int32_t accumulate) {
  cp_attn_desc d;
  d.heads_q = r->heads_q;
  d.heads_kv = r->heads_kv;
  d.len_q = r->chunk_len;
  d.len_kv = r->chunk_len;
  d.head_dim = r->head_dim;
  d.causal = r->causal;
  d.q_pos0 = (int64_t)r->rank * r->chunk_len;
  d.kv_pos0 = (int64_t)chunk * r->chunk_len;
  d.scale = r->scale;
  d.dtype = r->dtype;
  d.accumulate = accumulate;
  return d;
}

size_t elem_size(int32_t dtype) { return dtype == CP_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

int32_t cp_attn_abi_version(void) { return kAbiVersion; }

const char* cp_attn_status_string(int32_t status) {
  switch (status) {
    case CP_OK: return "ok";
    case CP_STEP_SKIPPED: return "step skipped: causally empty (no key visible to any query)";
    case CP_ERR_NULL: return "a required pointer is NULL";
    case CP_ERR_SHAPE: return "sizes or flags out of range or inconsistent";
    case CP_ERR_DTYPE: return "unknown dtype";
    case CP_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case CP_ERR_UNSUPPORTED: return "valid request not implemented by this build";
    case CP_ERR_HIP: return "HIP runtime error at launch";
    case CP_ERR_SCRATCH_LIMIT:
      return "request larger than the fixed scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

cp_status cp_attn_step(const cp_attn_desc* desc, const void* q, const void* k, const void* v,
                       float* o, float* lse, void* stream) {
  cp_status st = check_desc(desc);
  if (st != CP_OK) return st;
  if (desc->len_q == 0) return CP_OK;
  if (causally_empty(desc)) return CP_STEP_SKIPPED;
  if (desc->len_kv == 0) {
    st = check_ptrs({q, o, lse});
    if (st != CP_OK) return st;
    if (desc->accumulate) return CP_OK;  // nothing to fold in
  } else {
    st = check_ptrs({q, k, v, o, lse});
    if (st != CP_OK) return st;
  }
  cpa::StepParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.heads_q = desc->heads_q;
  p.heads_kv = desc->heads_kv;
  p.group = desc->heads_q / desc->heads_kv;
  p.len_q = desc->len_q;
  p.len_kv = desc->len_kv;
  p.head_dim = desc->head_dim;
  p.q_pos0 = desc->q_pos0;
  p.kv_pos0 = desc->kv_pos0;
  p.causal = desc->causal;
  p.accumulate = desc->accumulate;
  p.scale = resolve_scale(desc);
  p.scale_log2 = p.scale * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = desc->dtype == CP_BF16 ? cpa::launch_fwd_bf16(p, s) : cpa::launch_fwd_f32(p, s);
  return from_hip(e);
}

cp_status cp_attn_merge(int64_t rows, int32_t head_dim, float* o_acc, float* lse_acc,
                        const float* o, const float* lse, void* stream) {
  if (rows < 0 || rows > (int64_t)CP_MAX_HEADS * CP_MAX_LEN || head_dim < 1) return CP_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return CP_ERR_UNSUPPORTED;
  if (rows == 0) return CP_OK;
  cp_status st = check_ptrs({o_acc, lse_acc, o, lse});
  if (st != CP_OK) return st;
  return from_hip(cpa::launch_merge(rows, head_dim, o_acc, lse_acc, o, lse,
                                    static_cast<hipStream_t>(stream)));
}

cp_status cp_attn_bwd_prep(int64_t rows, int32_t head_dim, int32_t dtype, const float* o,
                           const void* d_o, float* delta, void* stream) {
  if (rows < 0 || rows > (int64_t)CP_MAX_HEADS * CP_MAX_LEN || head_dim < 1) return CP_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return CP_ERR_UNSUPPORTED;
  if (dtype != CP_F32 && dtype != CP_BF16) return CP_ERR_DTYPE;
  if (rows == 0) return CP_OK;
  cp_status st = check_ptrs({o, d_o, delta});
  if (st != CP_OK) return st;
  return from_hip(cpa::launch_bwd_prep(rows, head_dim, dtype == CP_BF16, o, d_o, delta,
                                       static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Shared body of the backward entry points. which: 1 = dK/dV, 2 = dQ, 3 = both.
cp_status bwd_impl(const cp_attn_desc* desc, const void* q, const void* k, const void* v,
                   const void* d_o, const float* lse, const float* delta, float* dq, float* dk,
                   float* dv, int which, void* stream) {
  cp_status st = check_desc(desc);
  if (st != CP_OK) return st;
  if (desc->dtype != CP_BF16) return CP_ERR_UNSUPPORTED;
  if (desc->len_q == 0 || desc->len_kv == 0) return CP_OK;
  if (causally_empty(desc)) return CP_STEP_SKIPPED;
  st = check_ptrs({q, k, v, d_o, lse, delta});
  if (st != CP_OK) return st;
  if (which & 1) {
    st = check_ptrs({dk, dv});
    if (st != CP_OK) return st;
  }
  if (which & 2) {
    st = check_ptrs({dq});
    if (st != CP_OK) return st;
  }
  cpa::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.d_o = d_o;
  p.lse = lse;
  p.delta = delta;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.heads_q = desc->heads_q;
  p.heads_kv = desc->heads_kv;
  p.group = desc->heads_q / desc->heads_kv;
  p.len_q = desc->len_q;
  p.len_kv = desc->len_kv;
  p.head_dim = desc->head_dim;
  p.q_pos0 = desc->q_pos0;
  p.kv_pos0 = desc->kv_pos0;
  p.causal = desc->causal;
  p.scale = resolve_scale(desc);
  p.scale_log2 = p.scale * 1.4426950408889634f;
  return from_hip(cpa::launch_bwd_bf16(p, which, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

cp_status cp_attn_bwd(const cp_attn_desc* desc, const void* q, const void* k, const void* v,
                      const void* d_o, const float* lse, const float* delta, float* dq,
                      float* dk, float* dv, void* stream) {
  return bwd_impl(desc, q, k, v, d_o, lse, delta, dq, dk, dv, 3, stream);
}

cp_status cp_attn_bwd_dkdv(const cp_attn_desc* desc, const void* q, const void* k,
                           const void* v, const void* d_o, const float* lse,
                           const float* delta, float* dk, float* dv, void* stream) {
  return bwd_impl(desc, q, k, v, d_o, lse, delta, nullptr, dk, dv, 1, stream);
}

cp_status cp_attn_bwd_dq(const cp_attn_desc* desc, const void* q, const void* k, const void* v,
                         const void* d_o, const float* lse, const float* delta, float* dq,
                         void* stream) {
  return bwd_impl(desc, q, k, v, d_o, lse, delta, dq, nullptr, nullptr, 2, stream);
}

int32_t cp_ring_schedule(int32_t n_cp, int32_t rank, int32_t causal, int32_t* chunks,
                         int32_t* classes) {
  if (!chunks || !classes) return CP_ERR_NULL;
  if (n_cp < 1 || n_cp > kMaxRing || rank < 0 || rank >= n_cp) return CP_ERR_SHAPE;
  if (causal != 0 && causal != 1) return CP_ERR_SHAPE;
  int32_t visited = 0;
  for (int32_t s = 0; s < n_cp; ++s) {
    const int32_t c = ((rank - s) % n_cp + n_cp) % n_cp;
    int32_t cls;
    if (!causal || c < rank) cls = 0;
    else if (c == rank) cls = 1;
    else cls = 2;
    chunks[s] = c;
    classes[s] = cls;
    if (cls != 2) ++visited;
  }
  return visited;
}

cp_status cp_attn_ring_fwd(const cp_ring_desc* ring, const void* q, const void* k_chunks,
                           const void* v_chunks, float* o, float* lse, float* o_work,
                           float* lse_work, void* stream) {
  cp_status st = check_ring(ring);
  if (st != CP_OK) return st;
  if ((o_work == nullptr) != (lse_work == nullptr)) return CP_ERR_NULL;
  const bool separate = o_work != nullptr;
  // Validate every step's descriptor up front so that an error writes nothing.
  cp_attn_desc d0 = ring_step_desc(ring, ring->rank, 0);
  st = check_desc(&d0);
  if (st != CP_OK) return st;
  st = check_ptrs({q, k_chunks, v_chunks, o, lse});
  if (st != CP_OK) return st;
  if (separate) {
    st = check_ptrs({o_work, lse_work});
    if (st != CP_OK) return st;
  }
  const size_t chunk_elems = (size_t)ring->heads_kv * ring->chunk_len * ring->head_dim;
  const size_t esz = elem_size(ring->dtype);
  const int64_t rows = (int64_t)ring->heads_q * ring->chunk_len;
  const char* kb = static_cast<const char*>(k_chunks);
  const char* vb = static_cast<const char*>(v_chunks);
  bool first = true;
  for (int32_t s = 0; s < ring->n_cp; ++s) {
    const int32_t c = ((ring->rank - s) % ring->n_cp + ring->n_cp) % ring->n_cp;
    if (ring->causal && c > ring->rank) continue;
    const void* kc = kb + (size_t)c * chunk_elems * esz;
    const void* vc = vb + (size_t)c * chunk_elems * esz;
    if (first) {
      cp_attn_desc d = ring_step_desc(ring, c, 0);
      st = cp_attn_step(&d, q, kc, vc, o, lse, stream);
      first = false;
    } else if (separate) {
      cp_attn_desc d = ring_step_desc(ring, c, 0);
      st = cp_attn_step(&d, q, kc, vc, o_work, lse_work, stream);
      if (st == CP_OK) st = cp_attn_merge(rows, ring->head_dim, o, lse, o_work, lse_work, stream);
    } else {
      cp_attn_desc d = ring_step_desc(ring, c, 1);
      st = cp_attn_step(&d, q, kc, vc, o, lse, stream);
    }
    if (st != CP_OK && st != CP_STEP_SKIPPED) return st;
  }
  return CP_OK;
}

cp_status cp_attn_ring_bwd(const cp_ring_desc* ring, const void* q, const void* k_chunks,
                           const void* v_chunks, const void* d_o, const float* o,
                           const float* lse, float* delta_work, float* dq, float* dk_chunks,
                           float* dv_chunks, void* stream) {
  cp_status st = check_ring(ring);
  if (st != CP_OK) return st;
  cp_attn_desc d0 = ring_step_desc(ring, ring->rank, 0);
  st = check_desc(&d0);
  if (st != CP_OK) return st;
  if (ring->dtype != CP_BF16) return CP_ERR_UNSUPPORTED;
  st = check_ptrs({q, k_chunks, v_chunks, d_o, o, lse, delta_work, dq, dk_chunks, dv_chunks});
  if (st != CP_OK) return st;
  const int64_t rows = (int64_t)ring->heads_q * ring->chunk_len;
  st = cp_attn_bwd_prep(rows, ring->head_dim, ring->dtype, o, d_o, delta_work, stream);
  if (st != CP_OK) return st;
  const size_t chunk_elems = (size_t)ring->heads_kv * ring->chunk_len * ring->head_dim;
  const size_t esz = elem_size(ring->dtype);
  const char* kb = static_cast<const char*>(k_chunks);
  const char* vb = static_cast<const char*>(v_chunks);
  for (int32_t s = 0; s < ring->n_cp; ++s) {
    const int32_t c = ((ring->rank - s) % ring->n_cp + ring->n_cp) % ring->n_cp;
    if (ring->causal && c > ring->rank) continue;
    cp_attn_desc d = ring_step_desc(ring, c, 0);
    st = cp_attn_bwd(&d, q, kb + (size_t)c * chunk_elems * esz, vb + (size_t)c * chunk_elems * esz,
                     d_o, lse, delta_work, dq, dk_chunks + (size_t)c * chunk_elems,
                     dv_chunks + (size_t)c * chunk_elems, stream);
    if (st != CP_OK && st != CP_STEP_SKIPPED) return st;
  }
  return CP_OK;
}

int32_t cp_zigzag_shards(int32_t n_cp, int32_t rank, int32_t* shards) {
  if (!shards) return CP_ERR_NULL;
  if (n_cp < 1 || n_cp > kMaxRing || rank < 0 || rank >= n_cp) return CP_ERR_SHAPE;
  shards[0] = rank;
  shards[1] = 2 * n_cp - 1 - rank;
  return 0;
}

cp_status cp_attn_ring_fwd_zigzag(const cp_ring_desc* ring, const void* q, const void* k_chunks,
                                  const void* v_chunks, float* o, float* lse, void* stream) {
  cp_status st = check_ring(ring);
  if (st != CP_OK) return st;
  cp_attn_desc d0 = ring_step_desc(ring, ring->rank, 0);
  st = check_desc(&d0);
  if (st != CP_OK) return st;
  st = check_ptrs({q, k_chunks, v_chunks, o, lse});
  if (st != CP_OK) return st;
  const int32_t n = ring->n_cp, lh = ring->chunk_len;
  const size_t esz = elem_size(ring->dtype);
  const size_t q_half = (size_t)ring->heads_q * lh * ring->head_dim;    // elements
  const size_t kv_half = (size_t)ring->heads_kv * lh * ring->head_dim;
  const int64_t rows_half = (int64_t)ring->heads_q * lh;
  const int32_t qs[2] = {ring->rank, 2 * n - 1 - ring->rank};
  bool started[2] = {false, false};
  for (int32_t s = 0; s < n; ++s) {
    const int32_t c = ((ring->rank - s) % n + n) % n;
    const int32_t ks[2] = {c, 2 * n - 1 - c};
    for (int a = 0; a < 2; ++a) {
      for (int b = 0; b < 2; ++b) {
        cp_attn_desc d = d0;
        d.q_pos0 = (int64_t)qs[a] * lh;
        d.kv_pos0 = (int64_t)ks[b] * lh;
        if (causally_empty(&d)) continue;
        d.accumulate = started[a] ? 1 : 0;
        const char* kb = static_cast<const char*>(k_chunks) + ((size_t)c * 2 + b) * kv_half * esz;
        const char* vb = static_cast<const char*>(v_chunks) + ((size_t)c * 2 + b) * kv_half * esz;
        st = cp_attn_step(&d, static_cast<const char*>(q) + a * q_half * esz, kb, vb,
                          o + a * q_half, lse + a * rows_half, stream);
        if (st != CP_OK && st != CP_STEP_SKIPPED) return st;
        started[a] = true;
      }
    }
  }
  return CP_OK;
}

cp_status cp_attn_ring_bwd_zigzag(const cp_ring_desc* ring, const void* q, const void* k_chunks,
                                  const void* v_chunks, const void* d_o, const float* o,
                                  const float* lse, float* delta_work, float* dq,
                                  float* dk_chunks, float* dv_chunks, void* stream) {
  cp_status st = check_ring(ring);
  if (st != CP_OK) return st;
  cp_attn_desc d0 = ring_step_desc(ring, ring->rank, 0);
  st = check_desc(&d0);
  if (st != CP_OK) return st;
  if (ring->dtype != CP_BF16) return CP_ERR_UNSUPPORTED;
  st = check_ptrs({q, k_chunks, v_chunks, d_o, o, lse, delta_work, dq, dk_chunks, dv_chunks});
  if (st != CP_OK) return st;
  const int32_t n = ring->n_cp, lh = ring->chunk_len;
  const size_t esz = elem_size(ring->dtype);
  const size_t q_half = (size_t)ring->heads_q * lh * ring->head_dim;
  const size_t kv_half = (size_t)ring->heads_kv * lh * ring->head_dim;
  const int64_t rows_half = (int64_t)ring->heads_q * lh;
  st = cp_attn_bwd_prep(2 * rows_half, ring->head_dim, ring->dtype, o, d_o, delta_work, stream);
  if (st != CP_OK) return st;
  const int32_t qs[2] = {ring->rank, 2 * n - 1 - ring->rank};
  for (int32_t s = 0; s < n; ++s) {
    const int32_t c = ((ring->rank - s) % n + n) % n;
    const int32_t ks[2] = {c, 2 * n - 1 - c};
    for (int a = 0; a < 2; ++a) {
      for (int b = 0; b < 2; ++b) {
        cp_attn_desc d = d0;
        d.q_pos0 = (int64_t)qs[a] * lh;
        d.kv_pos0 = (int64_t)ks[b] * lh;
        if (causally_empty(&d)) continue;
        const size_t kvo = ((size_t)c * 2 + b) * kv_half;
        st = cp_attn_bwd(&d, static_cast<const char*>(q) + a * q_half * esz,
                         static_cast<const char*>(k_chunks) + kvo * esz,
                         static_cast<const char*>(v_chunks) + kvo * esz,
                         static_cast<const char*>(d_o) + a * q_half * esz, lse + a * rows_half,
                         delta_work + a * rows_half, dq + a * q_half, dk_chunks + kvo,
                         dv_chunks + kvo, stream);
        if (st != CP_OK && st != CP_STEP_SKIPPED) return st;
      }
    }
  }
  return CP_OK;
}

// Striped ordering: stripe-local positions; the step with the chunk after the rank's own
// (c > rank) sees strictly earlier positions, hence kv_pos0 = 1.
cp_status cp_attn_ring_fwd_striped(const cp_ring_desc* ring, const void* q,
                                   const void* k_chunks, const void* v_chunks, float* o,
                                   float* lse, void* stream) {
  cp_status st = check_ring(ring);
  if (st != CP_OK) return st;
  cp_attn_desc d0 = ring_step_desc(ring, ring->rank, 0);
  st = check_desc(&d0);
  if (st != CP_OK) return st;
  st = check_ptrs({q, k_chunks, v_chunks, o, lse});
  if (st != CP_OK) return st;
  const size_t chunk = (size_t)ring->heads_kv * ring->chunk_len * ring->head_dim;
  const size_t esz = elem_size(ring->dtype);
  bool started = false;
  for (int32_t s = 0; s < ring->n_cp; ++s) {
    const int32_t c = ((ring->rank - s) % ring->n_cp + ring->n_cp) % ring->n_cp;
    cp_attn_desc d = d0;
    d.q_pos0 = 0;
    d.kv_pos0 = (ring->causal && c > ring->rank) ? 1 : 0;
    d.accumulate = started ? 1 : 0;
    st = cp_attn_step(&d, q, static_cast<const char*>(k_chunks) + c * chunk * esz,
                      static_cast<const char*>(v_chunks) + c * chunk * esz, o, lse, stream);
    if (st != CP_OK && st != CP_STEP_SKIPPED) return st;
    if (st == CP_OK) started = true;
  }
  return CP_OK;
}

cp_status cp_attn_ring_bwd_striped(const cp_ring_desc* ring, const void* q,
                                   const void* k_chunks, const void* v_chunks, const void* d_o,
                                   const float* o, const float* lse, float* delta_work,
                                   float* dq, float* dk_chunks, float* dv_chunks, void* stream) {
  cp_status st = check_ring(ring);
  if (st != CP_OK) return st;
  cp_attn_desc d0 = ring_step_desc(ring, ring->rank, 0);
  st = check_desc(&d0);
  if (st != CP_OK) return st;
  if (ring->dtype != CP_BF16) return CP_ERR_UNSUPPORTED;
  st = check_ptrs({q, k_chunks, v_chunks, d_o, o, lse, delta_work, dq, dk_chunks, dv_chunks});
  if (st != CP_OK) return st;
  const int64_t rows = (int64_t)ring->heads_q * ring->chunk_len;
  st = cp_attn_bwd_prep(rows, ring->head_dim, ring->dtype, o, d_o, delta_work, stream);
  if (st != CP_OK) return st;
  const size_t chunk = (size_t)ring->heads_kv * ring->chunk_len * ring->head_dim;
  const size_t esz = elem_size(ring->dtype);
  for (int32_t s = 0; s < ring->n_cp; ++s) {
    const int32_t c = ((ring->rank - s) % ring->n_cp + ring->n_cp) % ring->n_cp;
    cp_attn_desc d = d0;
    d.q_pos0 = 0;
    d.kv_pos0 = (ring->causal && c > ring->rank) ? 1 : 0;
    st = cp_attn_bwd(&d, q, static_cast<const char*>(k_chunks) + c * chunk * esz,
                     static_cast<const char*>(v_chunks) + c * chunk * esz, d_o, lse, delta_work,
                     dq, dk_chunks + c * chunk, dv_chunks + c * chunk, stream);
    if (st != CP_OK && st != CP_STEP_SKIPPED) return st;
  }
  return CP_OK;
}

}  // extern "C"
