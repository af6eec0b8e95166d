/*
 * cp_probe — device rate probes used beside the published peaks when reading a kernel's roofline.
 *
 * The attention step's contractions run on the matrix cores as v_mfma_f32_32x32x16_bf16 (bf16
 * inputs, fp32 accumulation). The published dense bf16 peak of an MI355X assumes every matrix
 * core busy at 2.4 GHz; what a device sustains under that load (clock, power) is lower. This call
 * launches a kernel that does nothing but those products, so a caller timing it (events on the
 * same stream) obtains the sustained rate: flops = workgroups * 4 wavefronts * iters * 4 * 32768.
 *
 * Conventions as in cp_attn.h: `sink` is device memory of workgroups * 256 floats that receives
 * one value per thread (so the products are not optimised away; its contents are meaningless);
 * `stream` is a hipStream_t (NULL = the null stream). Errors: CP_ERR_NULL for a NULL sink,
 * CP_ERR_SHAPE for workgroups or iters outside [1, 2^20]; nothing is launched then. The call
 * allocates nothing.
 */
#ifndef CP_PROBE_H
#define CP_PROBE_H

#include "cp_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue `workgroups` workgroups of 4 wavefronts; each wavefront issues iters * 4 independent
 * 32x32x16 bf16 MFMAs (four accumulators, so consecutive products never wait on each other). */
cp_status cp_probe_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream);

/* Copy n_float4 16-byte elements from src to dst (device memory, 16-byte aligned, not
 * overlapping): one load and one store per thread, as the library's HBM-bound elementwise
 * kernels do; 32 * n_float4 bytes move. Errors: CP_ERR_NULL, CP_ERR_ALIGN, CP_ERR_SHAPE for
 * n_float4 outside [1, 2^34]. */
cp_status cp_probe_copy(int64_t n_float4, const void* src, void* dst, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CP_PROBE_H */
