// One ring step of the backward (bf16 MFMA, fp32 accumulate): the gradient of
// loss = sum(O * dO) restricted to one key/value chunk, with P recomputed from the final
// forward LSE (P = exp(s - LSE)) rather than stored, and delta = rowsum(dO * O) from the prep
// kernel standing in for sum_j P_ij dP_ij.
//
// Workgroup kinds in one launch, no atomics (every output element has one owner):
//  * kv (dK part, dV part): a wave owns 32 keys of one key/value head (held in registers as MFMA
//    operands) and streams the query tiles of every query head of its group through LDS:
//      S = Q K^T, P = exp2(S*scale*log2e - LSE*log2e)         dV^T += dO^T P      (dV part)
//      S, P, dP = dO V^T, dS = P (dP - delta)                  dK^T += Q^T dS      (dK part)
//    (the group's heads summed in registers). With 4-wave workgroups a workgroup runs one part
//    on 128 keys; with 8-wave workgroups it runs both parts on 128 keys: waves 0-3 the dK
//    part, waves 4-7 the dV part, on the same keys and the same LDS tiles.
//  * dq: a wave owns 32 query rows of one head (128 or 256 rows per workgroup) and streams
//    key/value tiles:
//      S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T.
// Transposed operands (dO^T, Q^T, K^T) come from the same row-major LDS tiles through the
// LDS transpose read. Outputs are accumulated (+=) into fp32 dQ, dK, dV.
#include <math.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace cpa {
namespace {

constexpr int kQT = 64;    // query rows per tile (dkdv)
constexpr int kKT = 64;    // keys per tile (dq)
// Waves per workgroup (NW, a template parameter below): 4 or 8. Each wave owns 32 keys (kv
// parts) or 32 query rows (dQ part). With NW = 8 a kv workgroup covers 128 keys with both parts:
// waves 0-3 run the dK part and waves 4-7 the dV part on the same keys, so one LDS tile feeds
// both and each SIMD holds one wave of each kind; a dQ workgroup covers 256 rows. That halves the
// tile loads per product but leaves half as many workgroups to spread over the CUs: the launch
// takes 8 when the 8-wave grid still has kWideGrid workgroups or more (about eight per CU).
constexpr int kWideGrid = 2048;

// LDS operand reads issued ahead of their MFMA in the S/dP chains of the kv parts and of the
// dQ part (0 = compiler's choice). Measured on the 208K shard's backward ring: the dQ part
// gains ~7% at 2; the kv parts of the 8-wave launch lose 3% at 0 and 0.5% at 4 against 2
// (deeper dQ or accumulation prefetch spills registers).
#ifndef CP_BWD_PF_KV
#define CP_BWD_PF_KV 2
#endif
// The same for the transposed operands of the dK/dV/dQ accumulation products.
#ifndef CP_BWD_PF_ACC
#define CP_BWD_PF_ACC 0
#endif
#ifndef CP_BWD_PF_DQ
#define CP_BWD_PF_DQ 2
#endif

// Two MFMA chains acc_a += A_a[ks] * B_a[ks], acc_b += A_b[ks] * B_b[ks] over ks, with the A
// operands read from LDS PF steps ahead of their use (the reads of step ks + PF are issued
// before the MFMAs of step ks, and scheduling fences keep them there), so the LDS latency
// overlaps the matrix work. With PF = 0 the compiler schedules freely.
template <int KS, int PF, bool TWO, typename LA, typename LB>
__device__ __forceinline__ void mfma_chains(LA load_a, LB load_b, const u32x4_t* ba,
                                            const u32x4_t* bb, f32x16_t& acc_a, f32x16_t& acc_b) {
  if constexpr (PF == 0) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      acc_a = mfma32x32x16(load_a(ks), ba[ks], acc_a);
      if constexpr (TWO) acc_b = mfma32x32x16(load_b(ks), bb[ks], acc_b);
    }
  } else {
    u32x4_t ra[KS], rb[KS];
#pragma unroll
    for (int ks = 0; ks < PF; ++ks) {
      ra[ks] = load_a(ks);
      if constexpr (TWO) rb[ks] = load_b(ks);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + PF < KS) {
        ra[ks + PF] = load_a(ks + PF);
        if constexpr (TWO) rb[ks + PF] = load_b(ks + PF);
      }
      acc_a = mfma32x32x16(ra[ks], ba[ks], acc_a);
      if constexpr (TWO) acc_b = mfma32x32x16(rb[ks], bb[ks], acc_b);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// N MFMAs step(i, A_i) whose A operands are LDS reads load(i), issued PF steps ahead of their
// use behind scheduling fences (PF = 0: compiler's schedule).
template <int N, int PF, typename LA, typename ST>
__device__ __forceinline__ void mfma_pipe(LA load, ST step) {
  if constexpr (PF == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) step(i, load(i));
  } else {
    u32x4_t ra[N];
#pragma unroll
    for (int i = 0; i < PF && i < N; ++i) ra[i] = load(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (i + PF < N) ra[i + PF] = load(i + PF);
      step(i, ra[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// PART selects the products: kPartDV = S, P, dV^T += dO^T P (K operand only, LSE only);
// kPartDK = S, dP, dS, dK^T += Q^T dS (K and V operands, LSE and delta). Splitting dV from dK
// recomputes S once more but halves the accumulators, so each kernel runs two waves per SIMD.
constexpr int kPartDV = 1, kPartDK = 2;

// LDS of the kv parts: Q and dO tiles, double buffered, then LSE*log2e and delta per row.
template <int D>
constexpr int kv_smem_bytes() { return 2 * 2 * kQT * D * 2 + 2 * 2 * kQT * 4; }
// LDS of the dQ part: K and V tiles, double buffered (one such region per group of a split
// dQ workgroup).
template <int D>
constexpr int dq_smem_bytes() { return 2 * 2 * kKT * D * 2; }

// KW: waves that split the workgroup's keys (KW = NW, or NW / 2 when the two halves of the
// workgroup run the dK and the dV part on the same keys and share the tile loads).
template <int D, int PART, int NW, int KW = NW>
__device__ __forceinline__ void bwd_kv_body(const BwdParams& p, int w, char* smem) {
  constexpr int KS = D / 16, NB = D / 32, BNK = 32 * KW;
  constexpr bool DV = PART == kPartDV;
  uint16_t* const sq_base = reinterpret_cast<uint16_t*>(smem);
  uint16_t* const sdo_base = sq_base + 2 * kQT * D;
  float* const slse = reinterpret_cast<float*>(sdo_base + 2 * kQT * D);  // [2][kQT]
  float* const sdel = slse + 2 * kQT;                                     // [2][kQT]
  auto SQ = [&](int b) { return sq_base + b * (kQT * D); };
  auto SDO = [&](int b) { return sdo_base + b * (kQT * D); };

  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = tid >> 6;
  const int n_kt = (p.len_kv + BNK - 1) / BNK;
  const int g = w / n_kt;
  const int kt = w % n_kt;  // ascending: under causality the earliest keys have most work
  const int kv_base = kt * BNK;

  // This lane's key: column of the S = Q K^T and dP = dO V^T products.
  const int kwave = wave % KW;
  const int key = kv_base + 32 * kwave + col;
  const bool k_ok = key < p.len_kv;
  const int key_c = k_ok ? key : p.len_kv - 1;
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (size_t)g * p.len_kv * D;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + (size_t)g * p.len_kv * D;
  u32x4_t kb[KS], vb[DV ? 1 : KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4_t xk = *reinterpret_cast<const u32x4_t*>(kg + (size_t)key_c * D + 16 * ks + 8 * half);
    kb[ks] = k_ok ? xk : u32x4_t{0u, 0u, 0u, 0u};
    if constexpr (!DV) {
      const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(vg + (size_t)key_c * D + 16 * ks + 8 * half);
      vb[ks] = k_ok ? xv : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  // Query tiles that see at least one key of this workgroup.
  int qt_first = 0;
  if (p.causal) {
    const long long first_row = p.kv_pos0 + kv_base - p.q_pos0;
    qt_first = first_row <= 0 ? 0 : (int)min<long long>(first_row / kQT, (p.len_q + kQT - 1) / kQT);
  }
  const int n_qt = (p.len_q + kQT - 1) / kQT;
  const int per_head = n_qt - qt_first;
  const int n_it = per_head * p.group;

  f32x16_t acc[NB];  // dV^T or dK^T of the wave's 32 keys
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16_t{};

  using Dma = TileDma<D, kQT, 64 * NW>;
  // Issue the direct loads of tile `it` into LDS buffer `buf` and return this thread's staging
  // value for it: thread t < kQT fetches the LSE of row t (-inf past the end), thread kQT + t
  // (dK part) delta of row t. One value per thread, returned rather than written through a
  // capture, so that it stays in a register.
  // Tiles are visited head by head, query tiles in order: (head, tile) of the next tile to load
  // and of the tile being computed advance by one per iteration (no divisions in the loop).
  int ld_h = g * p.group, ld_qt = qt_first;
  int cur_qt = qt_first;
  auto load_it = [&](int it, int buf) -> float {
    (void)it;
    const int h = ld_h;
    const int q0 = ld_qt * kQT;
    if (++ld_qt == n_qt) {
      ld_qt = qt_first;
      ++ld_h;
    }
    const uint16_t* qh = static_cast<const uint16_t*>(p.q) + (size_t)h * p.len_q * D;
    const uint16_t* doh = static_cast<const uint16_t*>(p.d_o) + (size_t)h * p.len_q * D;
    Dma::issue_lean(qh, q0, p.len_q, SQ(buf), wave, lane);
    Dma::issue_lean(doh, q0, p.len_q, SDO(buf), wave, lane);
    const bool is_lse = tid < kQT;
    const int row = q0 + (is_lse ? tid : tid - kQT);
    float v = is_lse ? -INFINITY : 0.f;
    if (row < p.len_q && (is_lse || (!DV && tid < 2 * kQT))) {
      const float* src = is_lse ? p.lse : p.delta;
      v = src[(size_t)h * p.len_q + row];
    }
    return v;
  };
  // Publish a staged value; the LSE conversion happens here, after the tile's compute, so the
  // wait for the load is not paid up front. Rows past the end or with no visible key anywhere
  // get lse2 = +inf, hence P = 0.
  auto store_it = [&](int buf, float v) {
    const float l2 = v == -INFINITY ? INFINITY : v * kLog2e;
    if (tid < kQT) slse[buf * kQT + tid] = l2;
    else if (!DV && tid < 2 * kQT) sdel[buf * kQT + tid - kQT] = -v;  // dP starts at -delta
  };

  if (n_it > 0) store_it(0, load_it(0, 0));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const float c2 = p.scale_log2;
  const int dpos = causal_shift(p.q_pos0, p.kv_pos0);
  const int wave_key0 = kv_base + 32 * kwave;  // first key of the wave

  // Byte offsets of this lane's operand reads inside a tile. The swizzle of a row depends only on
  // its low four bits, so they are the same for every tile, buffer and 16-row step: computed
  // once and kept in registers (the empty asm keeps the compiler from recomputing the swizzle
  // in the loop); a read then costs one add for the buffer, the block being an immediate.
  uint32_t off_row[KS];  // row operand: row perm_row(col) of a 32-row block, chunk 2 ks + half
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    off_row[ks] = 2u * (uint32_t)tile_off<D>(perm_row(col), 2 * ks + half);
    asm volatile("" : "+v"(off_row[ks]));
  }
  uint32_t off_tr[2][NB];  // transposed operand (two reads): column block m of a 16-row step
  {
    const int g16 = lane >> 4, li = lane & 15;
    const int rr = 8 * (g16 >> 1) + (li >> 2);
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      const int cx = 32 * m + 16 * (g16 & 1) + 4 * (li & 3);
      off_tr[0][m] = 2u * (uint32_t)(tile_off<D>(rr, cx >> 3) + (cx & 7));
      off_tr[1][m] = 2u * (uint32_t)(tile_off<D>(rr + 4, cx >> 3) + (cx & 7));
      asm volatile("" : "+v"(off_tr[0][m]), "+v"(off_tr[1][m]));
    }
  }
  auto rd_row = [&](const uint16_t* tile, int b, int ks) {
    return *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(tile) +
                                             off_row[ks] + 64 * D * b);
  };
  auto rd_tr = [&](const uint16_t* tile, int r0, int m) {  // rows r0 .. r0 + 15, r0 % 16 == 0
    const char* t = reinterpret_cast<const char*>(tile) + 2 * r0 * D;
    const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(t + off_tr[0][m]));
    const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(t + off_tr[1][m]));
    const u32x2_t w0 = __builtin_bit_cast(u32x2_t, v0);
    const u32x2_t w1 = __builtin_bit_cast(u32x2_t, v1);
    return u32x4_t{w0[0], w0[1], w1[0], w1[1]};
  };

  for (int it = 0; it < n_it; ++it) {
    const int buf = it & 1;
    float stg = 0.f;
    if (it + 1 < n_it) stg = load_it(it + 1, buf ^ 1);
    const int q0 = cur_qt * kQT;
    if (++cur_qt == n_qt) cur_qt = qt_first;
    // One 32-row block of the tile against the wave's 32 keys, in three steps:
    // chains: S = Q K^T (and dP = dO V^T) on the matrix cores;
    auto chains = [&](int b, f32x16_t& s, f32x16_t& dp, auto pf) {
      s = f32x16_t{};
      dp = f32x16_t{};
      if constexpr (!DV) {
        // dP accumulates onto -delta of its rows, so that dS = P * dP needs no subtraction
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int rbase = 32 * b + 16 * (a4 >> 1) + 8 * half + 4 * (a4 & 1);
          const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(sdel + buf * kQT + rbase);
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[4 * a4 + e] = d4[e];
        }
      }
      mfma_chains<KS, decltype(pf)::value, !DV>(
          [&](int ks) { return rd_row(SQ(buf), b, ks); },
          [&](int ks) { return rd_row(SDO(buf), b, ks); }, kb, vb, s, dp);
    };
    // soft: P = exp2(S*c - lse2) (dV part) or dS = P (dP - delta) (dK part), to bf16;
    auto soft = [&](int b, const f32x16_t& s, const f32x16_t& dp, bool need_mask,
                    u32x4_t (&pb)[2]) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        // accumulator registers 4*a4 .. 4*a4+3 hold 4 consecutive query rows of the tile
        const int rbase = 32 * b + 16 * (a4 >> 1) + 8 * half + 4 * (a4 & 1);
        float v4[4];
        const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(slse + buf * kQT + rbase);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * a4 + e], c2, -l4[e]));
          if (need_mask && key - (q0 + rbase + e) > dpos) pr = 0.f;
          if constexpr (DV) v4[e] = pr;
          else v4[e] = pr * dp[4 * a4 + e];  // P (dP - delta)
        }
        pb[a4 >> 1][2 * (a4 & 1)] = pack_bf16x2(v4[0], v4[1]);
        pb[a4 >> 1][2 * (a4 & 1) + 1] = pack_bf16x2(v4[2], v4[3]);
      }
    };
    // accum: dV^T += dO^T P or dK^T += Q^T dS (transposed operand via the transpose read).
    auto accum = [&](int b, const u32x4_t (&pb)[2]) {
      const uint16_t* tt = DV ? SDO(buf) : SQ(buf);
      mfma_pipe<2 * NB, CP_BWD_PF_ACC>(
          [&](int i) { return rd_tr(tt, 32 * b + 16 * (i / NB), i % NB); },
          [&](int i, const u32x4_t& a) { acc[i % NB] = mfma32x32x16(a, pb[i / NB], acc[i % NB]); });
    };
    auto do_block = [&](int b, bool need_mask) {
      f32x16_t s, dp;
      u32x4_t pb[2];
      chains(b, s, dp, std::integral_constant<int, CP_BWD_PF_KV>{});
      soft(b, s, dp, need_mask, pb);
      accum(b, pb);
    };
    if (!p.causal || wave_key0 + 31 - q0 <= dpos) {
      // every key of the wave is visible to every row of the tile: no mask, no branches
      if constexpr (DV) {
        // the dV part has one S chain per block: run the two blocks' chains interleaved, so that
        // consecutive MFMAs never wait for each other's accumulator
        f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{}, unused = f32x16_t{};
        u32x4_t pb0[2], pb1[2];
        mfma_chains<KS, CP_BWD_PF_KV, true>(
            [&](int ks) { return rd_row(SQ(buf), 0, ks); },
            [&](int ks) { return rd_row(SQ(buf), 1, ks); }, kb,
            kb, s0, s1);
        soft(0, s0, unused, false, pb0);
        soft(1, s1, unused, false, pb1);
        accum(0, pb0);
        accum(1, pb1);
      } else {
        do_block(0, false);
        do_block(1, false);
      }
    } else {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int brow = q0 + 32 * b;  // first row of the block
        // no row of the block sees the wave's first key: nothing to do
        if (wave_key0 - (brow + 31) > dpos) continue;
        // some key of the wave invisible to the block's first row: mask
        do_block(b, wave_key0 + 31 - brow > dpos);
      }
    }
    if (it + 1 < n_it) store_it(buf ^ 1, stg);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (!k_ok) return;
  float* out = (DV ? p.dv : p.dk) + ((size_t)g * p.len_kv + key) * D;
  const float f = DV ? 1.f : p.scale;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      f32x4_t* ptr = reinterpret_cast<f32x4_t*>(out + 32 * nb + 8 * a4 + 4 * half);
      f32x4_t o4 = *ptr;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] += f * acc[nb][4 * a4 + e];
      *ptr = o4;
    }
}

// SPLIT (8-wave workgroups only): the workgroup takes half of work item w / 2, rows
// [128 (w % 2), 128 (w % 2) + 128) of its 256, and its two groups of four waves split the keys:
// group A the first ceil(n/2) tiles, group B the rest, each streaming its own tiles through its
// own LDS region; B hands its partial dQ to A through LDS at the end. Such workgroups take half
// as long, and the launch ends with them.
template <int D, int NW, bool SPLIT = false>
__device__ __forceinline__ void bwd_dq_body(const BwdParams& p, int w, char* smem) {
  static_assert(!SPLIT || NW == 8, "a split dQ workgroup is two groups of four waves");
  constexpr int KS = D / 16, NB = D / 32, BM = 32 * NW;
  constexpr int RW = SPLIT ? 4 : NW;  // waves that share the key tiles (and own the rows)
  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = tid >> 6;
  const int grp = SPLIT ? __builtin_amdgcn_readfirstlane(wave >> 2) : 0;  // wave-uniform
  const int wv = SPLIT ? wave & 3 : wave;  // wave within the group
  uint16_t* const sk_base = reinterpret_cast<uint16_t*>(smem) + grp * (4 * kKT * D);
  uint16_t* const sv_base = sk_base + 2 * kKT * D;
  auto SK = [&](int b) { return sk_base + b * (kKT * D); };
  auto SV = [&](int b) { return sv_base + b * (kKT * D); };

  const int u = SPLIT ? w >> 1 : w;  // work item of 256 (8 waves) or 128 (4 waves) rows
  const int n_qt = (p.len_q + BM - 1) / BM;
  const int h_in = u % p.group;
  const int rest = u / p.group;
  const int qt = n_qt - 1 - rest % n_qt;  // causally longest tiles first
  const int g = rest / n_qt;
  const int h = g * p.group + h_in;
  const int q_base = qt * BM + (SPLIT ? 32 * RW * (w & 1) : 0);

  const int qi = q_base + 32 * wv + col;
  const bool q_ok = qi < p.len_q;
  const int qi_c = q_ok ? qi : p.len_q - 1;
  const uint16_t* qh = static_cast<const uint16_t*>(p.q) + (size_t)h * p.len_q * D;
  const uint16_t* doh = static_cast<const uint16_t*>(p.d_o) + (size_t)h * p.len_q * D;
  u32x4_t qb[KS], dob[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4_t xq = *reinterpret_cast<const u32x4_t*>(qh + (size_t)qi_c * D + 16 * ks + 8 * half);
    const u32x4_t xd = *reinterpret_cast<const u32x4_t*>(doh + (size_t)qi_c * D + 16 * ks + 8 * half);
    qb[ks] = q_ok ? xq : u32x4_t{0u, 0u, 0u, 0u};
    dob[ks] = q_ok ? xd : u32x4_t{0u, 0u, 0u, 0u};
  }
  const float lse_raw = q_ok ? p.lse[(size_t)h * p.len_q + qi] : -INFINITY;
  const float lse2 = lse_raw == -INFINITY ? INFINITY : lse_raw * kLog2e;
  const float del = q_ok ? p.delta[(size_t)h * p.len_q + qi] : 0.f;

  const int last_row = min(q_base + 32 * RW, p.len_q) - 1;
  long long nk = p.len_kv;
  if (p.causal) nk = min(nk, p.q_pos0 + last_row - p.kv_pos0 + 1);
  const int n_kt = nk > 0 ? (int)((nk + kKT - 1) / kKT) : 0;
  // This group's key tiles [kt0, kt_end); a split workgroup's groups step through n_steps
  // tiles each (group B idles through the last one when n_kt is odd).
  const int n_steps = SPLIT ? (n_kt + 1) / 2 : n_kt;
  const int kt0 = grp == 0 ? 0 : n_steps;
  const int kt_end = grp == 0 ? n_steps : n_kt;

  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (size_t)g * p.len_kv * D;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + (size_t)g * p.len_kv * D;
  using Dma = TileDma<D, kKT, 64 * RW>;

  f32x16_t dqt[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) dqt[nb] = f32x16_t{};

  if (kt0 < kt_end) {
    Dma::issue(kg, kt0 * kKT, p.len_kv, SK(0), wv, lane);
    Dma::issue(vg, kt0 * kKT, p.len_kv, SV(0), wv, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const float c2 = p.scale_log2;
  const int dpos = causal_shift(p.q_pos0, p.kv_pos0);
  const int wave_row0 = q_base + 32 * wv;

  // Key tiles that every row of the workgroup sees in full (and that lie inside the chunk) come
  // first: they run without any mask code. The rest (the diagonal and the ragged end) follow.
  int n_full = p.len_kv / kKT;
  if (p.causal) {
    const long long lim = (long long)dpos + q_base + 1;  // keys < lim visible to row q_base
    n_full = (int)max(0LL, min<long long>(n_full, lim / kKT));
  }
  n_full = min(n_full, n_kt);

  // `bufc` = (kt - kt0) % 2 as a compile-time constant where the caller knows it (then every
  // LDS address of the tile is a per-lane base plus an immediate offset), or -1.
  auto tile = [&](int kt, auto fullc, auto bufc) {
    constexpr bool kFull = decltype(fullc)::value;
    const int buf = decltype(bufc)::value < 0 ? ((kt - kt0) & 1) : decltype(bufc)::value;
    if (kt + 1 < kt_end) {
      Dma::issue(kg, (kt + 1) * kKT, p.len_kv, SK(buf ^ 1), wv, lane);
      Dma::issue(vg, (kt + 1) * kKT, p.len_kv, SV(buf ^ 1), wv, lane);
    }
    const int key0 = kt * kKT;
    // One 32-key block of the tile against the wave's 32 query rows.
    auto do_block = [&](int blk, bool need_mask) {
      // dP^T accumulates onto -delta of the lane's row, so that dS^T = P^T * dP^T
      f32x16_t s = f32x16_t{}, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = -del;
      const int arow = 32 * blk + perm_row(col);
      mfma_chains<KS, CP_BWD_PF_DQ, true>(  // S^T and dP^T chains interleaved
          [&](int ks) { return tile_row8<D>(SK(buf), arow, 2 * ks + half); },
          [&](int ks) { return tile_row8<D>(SV(buf), arow, 2 * ks + half); }, qb, dob, s, dp);
      // Accumulator register r holds key key0 + 32 blk + 8 half + koff(r) (rows loaded through
      // perm_row), with koff(r) = (r & 7) + 16 (r >> 3); it is visible iff koff(r) <= klim.
      int klim = 0;
      if (need_mask) {
        const int kb0 = key0 + 32 * blk + 8 * half;
        klim = p.len_kv - 1 - kb0;
        if (p.causal) klim = min(klim, qi + dpos - kb0);
      }
      u32x4_t dsb[2];
#pragma unroll
      for (int r2 = 0; r2 < 8; ++r2) {
        float dsv[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * r2 + e;
          float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c2, -lse2));
          if (need_mask && (r & 7) + 16 * (r >> 3) > klim) pr = 0.f;
          dsv[e] = pr * dp[r];
        }
        dsb[r2 >> 2][r2 & 3] = pack_bf16x2(dsv[0], dsv[1]);
      }
      mfma_pipe<2 * NB, CP_BWD_PF_ACC>(
          [&](int i) { return tile_col8<D>(SK(buf), 32 * blk + 16 * (i / NB), 32 * (i % NB), lane); },
          [&](int i, const u32x4_t& a) { dqt[i % NB] = mfma32x32x16(a, dsb[i / NB], dqt[i % NB]); });
    };
    if constexpr (kFull) {
      do_block(0, false);
      do_block(1, false);
    } else {
      const bool need_mask =
          key0 + kKT > p.len_kv || (p.causal && key0 + kKT - 1 - wave_row0 > dpos);
      if (!p.causal || key0 - (wave_row0 + 31) <= dpos) {
        do_block(0, need_mask);
        do_block(1, need_mask);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  if constexpr (!SPLIT) {
    int kt = 0;
    for (; kt + 1 < n_full; kt += 2) {  // unrolled by two: the buffer index is a constant
      tile(kt, std::true_type{}, std::integral_constant<int, 0>{});
      tile(kt + 1, std::true_type{}, std::integral_constant<int, 1>{});
    }
    for (; kt < n_kt; ++kt) tile(kt, std::bool_constant<false>{}, std::integral_constant<int, -1>{});
  } else {
    const int cnt = kt_end - kt0;
    const int nf = max(0, min(cnt, n_full - kt0));  // this group's mask-free tiles come first
    int i = 0;
    for (; i + 1 < nf; i += 2) {
      tile(kt0 + i, std::true_type{}, std::integral_constant<int, 0>{});
      tile(kt0 + i + 1, std::true_type{}, std::integral_constant<int, 1>{});
    }
    for (; i < cnt; ++i) tile(kt0 + i, std::bool_constant<false>{}, std::integral_constant<int, -1>{});
    for (; i < n_steps; ++i) __syncthreads();  // group B, one tile fewer: keeps step with A
    // B's partial dQ^T goes to A through LDS (the tiles are no longer read), lane-contiguous.
    float* const xch = reinterpret_cast<float*>(smem) + wv * (16 * NB) * 64;
    if (grp == 1) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[(16 * nb + r) * 64 + lane] = dqt[nb][r];
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) dqt[nb][r] += xch[(16 * nb + r) * 64 + lane];
  }

  if (!q_ok) return;
  float* dqr = p.dq + ((size_t)h * p.len_q + qi) * D;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      f32x4_t* ptr = reinterpret_cast<f32x4_t*>(dqr + 32 * nb + 8 * a4 + 4 * half);
      f32x4_t o4 = *ptr;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] += p.scale * dqt[nb][4 * a4 + e];
      *ptr = o4;
    }
}

// One launch per ring step: the dK part's workgroups first (the longest), then the dV part's,
// then the dQ kernel's, so that the short dQ workgroups fill the tail left by the others, and
// last the split dQ workgroups (8-wave launches), which take half as long again and so even out
// the launch's end. The bodies share one LDS buffer; n_dk, n_dv, n_dq, n_dqs are the segment
// sizes (0 = segment off). With NW = 8 the first segment holds the mixed dK/dV workgroups and
// the second is empty.
template <int D, int NW>
__global__ void __launch_bounds__(64 * NW, 2)
    bwd_kernel(BwdParams p, int n_dk, int n_dv, int n_dq, int n_dqs) {
  constexpr int kDq = (NW == 8 ? 2 : 1) * dq_smem_bytes<D>();
  constexpr int kSmem = kv_smem_bytes<D>() > kDq ? kv_smem_bytes<D>() : kDq;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  int b = blockIdx.x;
  if (b < n_dk) {
    if constexpr (NW == 8) {
      // waves 0-3: dK part, waves 4-7: dV part, same 128 keys, shared tiles
      if ((threadIdx.x >> 6) < 4)
        bwd_kv_body<D, kPartDK, NW, 4>(p, xcd_remap(b, n_dk), smem);
      else
        bwd_kv_body<D, kPartDV, NW, 4>(p, xcd_remap(b, n_dk), smem);
    } else {
      bwd_kv_body<D, kPartDK, NW>(p, xcd_remap(b, n_dk), smem);
    }
    return;
  }
  b -= n_dk;
  if (b < n_dv) {
    bwd_kv_body<D, kPartDV, NW>(p, xcd_remap(b, n_dv), smem);
    return;
  }
  b -= n_dv;
  if (b < n_dq) {
    bwd_dq_body<D, NW>(p, xcd_remap(b, n_dq), smem);
    return;
  }
  b -= n_dq;
  if constexpr (NW == 8) {
    // halves of the work items that follow the n_dq whole ones
    if (b < n_dqs) bwd_dq_body<D, NW, true>(p, 2 * n_dq + xcd_remap(b, n_dqs), smem);
  }
}

// Workgroups of the launch at NW waves: {dK part, dV part, dQ part, split dQ part}.
struct BwdGrid {
  int n_dk, n_dv, n_dq, n_dqs;
  long long total() const { return (long long)n_dk + n_dv + n_dq + n_dqs; }
};
BwdGrid bwd_grid(const BwdParams& p, int which, int nw) {
  const int rows = 32 * nw;
  const int n_q = ((p.len_q + rows - 1) / rows) * p.heads_q;
  if (nw == 8) {  // one workgroup per 128 keys for both parts
    const int n_mix = ((p.len_kv + 127) / 128) * p.heads_kv;
    return {(which & 1) ? n_mix : 0, 0, (which & 2) ? n_q : 0, 0};
  }
  const int n_kv = ((p.len_kv + rows - 1) / rows) * p.heads_kv;
  return {(which & 1) ? n_kv : 0, (which & 1) ? n_kv : 0, (which & 2) ? n_q : 0, 0};
}

template <int D, int NW>
hipError_t launch_dn(const BwdParams& p, const BwdGrid& g, hipStream_t s) {
  hipLaunchKernelGGL((bwd_kernel<D, NW>), dim3((unsigned)g.total()), dim3(64 * NW), 0, s, p,
                     g.n_dk, g.n_dv, g.n_dq, g.n_dqs);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdParams& p, int which, hipStream_t s) {
  BwdGrid wide = bwd_grid(p, which, 8);
  if (wide.total() == 0) return hipSuccess;
  if (wide.total() >= kWideGrid) {
    // When every key is visible to every row, all dQ work items take the same time and the
    // launch would end on a ragged last round of them: the last round's worth (one item per
    // CU) runs as split workgroups of half the length instead. (Under a causal mask the items
    // are ordered longest first and the short ones already even out the end.)
    const bool uniform = !p.causal || p.kv_pos0 + p.len_kv - 1 <= p.q_pos0;
    const int tail = uniform ? min(wide.n_dq, device_cus()) : 0;
    wide.n_dq -= tail;
    wide.n_dqs = 2 * tail;
    return launch_dn<D, 8>(p, wide, s);
  }
  return launch_dn<D, 4>(p, bwd_grid(p, which, 4), s);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, int which, hipStream_t s) {
  if (p.head_dim == 128) return launch_d<128>(p, which, s);
  if (p.head_dim == 64) return launch_d<64>(p, which, s);
  return hipErrorInvalidValue;
}

}  // namespace cpa
