/*
 * cp_fir — the context-parallel causal FIR convolution of StripedHyena 2's short and medium
 * convolutions, one GPU's share, on an AMD MI355X (gfx950).
 *
 * The method (StripedHyena 2 context-parallelism page, section 3, the p2p convolution bullet):
 * the sequence [D, L] is cut along its length into N_cp shards [D, Lc] (section 1 of the same
 * page). Every channel c is convolved causally with its own filter h[c, 0 .. l_h - 1]:
 *     y[c, t] = sum_k h[c, k] * x[c, t - k]    (x = 0 before the start of the sequence).
 * Because the filter is finite, a shard's outputs need only its own samples except the first
 * l_h - 1, which also need the last l_h - 1 samples of the previous shard (the halo). The same
 * section proposes overlapping the halo exchange with compute: convolve the shard with zero
 * history first, then add the boundary terms when the halo has arrived. These calls are those
 * two stages plus the sender's side (packing the tail that goes to the next rank).
 *
 * Conventions (as in cp_attn.h unless stated): device pointers, 16-byte aligned, row-major,
 * time innermost. x [channels, shard_len] and h [channels, taps] in `dtype` (CP_BF16 or CP_F32);
 * halo [channels, taps - 1] in `dtype`; y [channels, shard_len] fp32, accumulation in fp32.
 * Limits: 1 <= taps <= CP_FIR_MAX_TAPS and taps - 1 <= shard_len (the halo comes from one
 * neighbour); channels <= CP_FIR_MAX_CHANNELS; shard_len <= CP_MAX_LEN. Errors are reported
 * before anything is enqueued; the library allocates nothing.
 */
#ifndef CP_FIR_H
#define CP_FIR_H

#include "cp_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

#define CP_FIR_MAX_TAPS 1024
#define CP_FIR_MAX_CHANNELS (1 << 20)

typedef struct {
  int32_t channels;   /* D */
  int32_t shard_len;  /* Lc: samples per shard */
  int32_t taps;       /* l_h */
  int32_t dtype;      /* cp_dtype of x, h and halo */
} cp_fir_desc;

/* cp_fir_local — stage one: y = causal convolution of the shard x with zero history
 * (overwrites y). Independent of the halo, so it can run while the halo is in flight. */
cp_status cp_fir_local(const cp_fir_desc* desc, const void* x, const void* h, float* y,
                       void* stream);

/* cp_fir_pack_halo — the sender's side: halo = the last taps - 1 samples of every channel of x,
 * i.e. the [channels, taps - 1] message for the next rank. taps == 1: nothing to do. */
cp_status cp_fir_pack_halo(const cp_fir_desc* desc, const void* x, void* halo, void* stream);

/* cp_fir_halo — stage two: y[c, i] += sum_{k > i} h[c, k] * halo[c, taps - 1 + i - k] for
 * i < taps - 1, the boundary terms that the previous shard's tail contributes. Run after
 * cp_fir_local on the same y (same stream, or ordered by the caller). */
cp_status cp_fir_halo(const cp_fir_desc* desc, const void* halo, const void* h, float* y,
                      void* stream);

/* cp_fir_ring — all n_cp shards of one sequence on this GPU: x_shards, y_shards
 * [n_cp, channels, shard_len] (shard r holds samples r*Lc .. r*Lc + Lc - 1); halo_work
 * [n_cp, channels, taps - 1] in `dtype` is caller-provided scratch (may be NULL when taps == 1).
 * Packs every shard's tail, runs the local stage on every shard, then adds shard r - 1's tail
 * into shard r (shard 0 has zero history). */
cp_status cp_fir_ring(const cp_fir_desc* desc, int32_t n_cp, const void* x_shards,
                      const void* h, void* halo_work, float* y_shards, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CP_FIR_H */
