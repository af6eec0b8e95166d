// A plain C++ consumer of the library's C ABI (no Python, no torch): reads one rank's bf16 ring
// inputs from a file, runs cp_attn_ring_fwd and cp_attn_ring_bwd on device buffers it allocates
// itself, and writes the fp32 results back to a file. Used by tests/test_c_abi_gpu.py.
//
// Input file: int32 header {heads_q, heads_kv, chunk_len, head_dim, n_cp, rank, causal}, then
// bf16 q [heads_q, Lc, d], k [n_cp, heads_kv, Lc, d], v (same), d_o [heads_q, Lc, d].
// Output file: fp32 o [heads_q, Lc, d], lse [heads_q, Lc], dq [heads_q, Lc, d],
// dk [n_cp, heads_kv, Lc, d], dv (same).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "cp_attn.h"

static bool hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return false;
  }
  return true;
}

static bool cp_ok(cp_status s, const char* what) {
  if (s != CP_OK) {
    std::fprintf(stderr, "%s: %s\n", what, cp_attn_status_string(s));
    return false;
  }
  return true;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s INPUT OUTPUT\n", argv[0]);
    return 2;
  }
  FILE* fi = std::fopen(argv[1], "rb");
  if (!fi) return 2;
  int32_t h[7];
  if (std::fread(h, sizeof(int32_t), 7, fi) != 7) return 2;
  const int32_t hq = h[0], hkv = h[1], lc = h[2], d = h[3], n_cp = h[4], rank = h[5];
  const size_t nq = (size_t)hq * lc * d, nkv = (size_t)n_cp * hkv * lc * d, nrow = (size_t)hq * lc;
  std::vector<uint16_t> q(nq), k(nkv), v(nkv), d_o(nq);
  if (std::fread(q.data(), 2, nq, fi) != nq || std::fread(k.data(), 2, nkv, fi) != nkv ||
      std::fread(v.data(), 2, nkv, fi) != nkv || std::fread(d_o.data(), 2, nq, fi) != nq)
    return 2;
  std::fclose(fi);

  cp_ring_desc ring = {};
  ring.heads_q = hq;
  ring.heads_kv = hkv;
  ring.chunk_len = lc;
  ring.head_dim = d;
  ring.n_cp = n_cp;
  ring.rank = rank;
  ring.causal = h[6];
  ring.scale = 0.f;  // 1/sqrt(d)
  ring.dtype = CP_BF16;

  void *dq_in = nullptr, *dk_in = nullptr, *dv_in = nullptr, *ddo = nullptr;
  float *o = nullptr, *lse = nullptr, *delta = nullptr, *dq = nullptr, *dk = nullptr, *dv = nullptr;
  bool ok = hip_ok(hipMalloc(&dq_in, nq * 2), "hipMalloc") &&
            hip_ok(hipMalloc(&dk_in, nkv * 2), "hipMalloc") &&
            hip_ok(hipMalloc(&dv_in, nkv * 2), "hipMalloc") &&
            hip_ok(hipMalloc(&ddo, nq * 2), "hipMalloc") &&
            hip_ok(hipMalloc(&o, nq * 4), "hipMalloc") &&
            hip_ok(hipMalloc(&lse, nrow * 4), "hipMalloc") &&
            hip_ok(hipMalloc(&delta, nrow * 4), "hipMalloc") &&
            hip_ok(hipMalloc(&dq, nq * 4), "hipMalloc") &&
            hip_ok(hipMalloc(&dk, nkv * 4), "hipMalloc") &&
            hip_ok(hipMalloc(&dv, nkv * 4), "hipMalloc");
  ok = ok && hip_ok(hipMemcpy(dq_in, q.data(), nq * 2, hipMemcpyHostToDevice), "copy q") &&
       hip_ok(hipMemcpy(dk_in, k.data(), nkv * 2, hipMemcpyHostToDevice), "copy k") &&
       hip_ok(hipMemcpy(dv_in, v.data(), nkv * 2, hipMemcpyHostToDevice), "copy v") &&
       hip_ok(hipMemcpy(ddo, d_o.data(), nq * 2, hipMemcpyHostToDevice), "copy do") &&
       hip_ok(hipMemset(dq, 0, nq * 4), "zero dq") && hip_ok(hipMemset(dk, 0, nkv * 4), "zero dk") &&
       hip_ok(hipMemset(dv, 0, nkv * 4), "zero dv");
  ok = ok && cp_ok(cp_attn_ring_fwd(&ring, dq_in, dk_in, dv_in, o, lse, nullptr, nullptr, nullptr),
                   "cp_attn_ring_fwd");
  ok = ok && cp_ok(cp_attn_ring_bwd(&ring, dq_in, dk_in, dv_in, ddo, o, lse, delta, dq, dk, dv,
                                    nullptr),
                   "cp_attn_ring_bwd");
  ok = ok && hip_ok(hipDeviceSynchronize(), "synchronize");

  std::vector<float> ho(nq), hl(nrow), hdq(nq), hdk(nkv), hdv(nkv);
  ok = ok && hip_ok(hipMemcpy(ho.data(), o, nq * 4, hipMemcpyDeviceToHost), "copy o") &&
       hip_ok(hipMemcpy(hl.data(), lse, nrow * 4, hipMemcpyDeviceToHost), "copy lse") &&
       hip_ok(hipMemcpy(hdq.data(), dq, nq * 4, hipMemcpyDeviceToHost), "copy dq") &&
       hip_ok(hipMemcpy(hdk.data(), dk, nkv * 4, hipMemcpyDeviceToHost), "copy dk") &&
       hip_ok(hipMemcpy(hdv.data(), dv, nkv * 4, hipMemcpyDeviceToHost), "copy dv");
  for (void* p : {dq_in, dk_in, dv_in, ddo}) hipFree(p);
  for (float* p : {o, lse, delta, dq, dk, dv}) hipFree(p);
  if (!ok) return 1;

  FILE* fo = std::fopen(argv[2], "wb");
  if (!fo) return 2;
  std::fwrite(ho.data(), 4, nq, fo);
  std::fwrite(hl.data(), 4, nrow, fo);
  std::fwrite(hdq.data(), 4, nq, fo);
  std::fwrite(hdk.data(), 4, nkv, fo);
  std::fwrite(hdv.data(), 4, nkv, fo);
  std::fclose(fo);
  std::printf("ok: rank %d of %d, %d/%d heads, %d rows, d %d\n", rank, n_cp, hq, hkv, lc, d);
  return 0;
}
