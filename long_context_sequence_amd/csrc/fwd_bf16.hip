// One ring step of the forward on gfx950: the rank's query tile against one key/value chunk,
// bf16 MFMA for both contractions, online softmax in registers (StripedHyena 2
// context-parallelism page, section 2, ring attention steps 2-3).
//
// Work decomposition
//   workgroup = NW waves = one query head x BM = 32*NW query rows; each wave owns 32 rows.
//   Keys stream through LDS in tiles of 64 (double buffered), K and V both row-major.
//
// Register-level formulation (per wave, per 64-key tile)
//   S^T[key][query] = K Q^T      A = K rows from LDS, B = the wave's Q rows held in registers
//   P^T = exp2(S^T * scale*log2e - m)
//   O^T[d][query] += V^T P^T     A = V^T rows from LDS, B = P^T straight from the S^T
//                                accumulator registers (no LDS round trip for P)
// With S^T, each lane's accumulator column is one query row, so the row max needs one swap with
// the lane 32 apart, the row sum stays lane-local until the end and the O rescale is one scalar
// per lane. Loading K row perm_row(m) for MFMA row m makes every run of 8 accumulator registers
// cover 8 consecutive keys, so the matching V^T operand is one transpose read (two
// ds_read_b64_tr_b16) of the row-major V tile.
//
// Causality: the workgroup visits only tiles some of its rows can see; the mask is applied only
// on tiles that straddle the diagonal (for the wave's rows) or the ragged end of the chunk.
// Pipelining: S of the next tile is computed on the matrix cores while the VALU turns the
// current tile's S into P, so each wave keeps both busy.
#include <math.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace cpa {
namespace {

// Launch shape: waves per workgroup (32 query rows each) and keys per LDS tile.
#ifndef CP_FWD_WAVES
#define CP_FWD_WAVES 4
#endif
#ifndef CP_FWD_KEYS
#define CP_FWD_KEYS 64
#endif
#ifndef CP_FWD_OCC
#define CP_FWD_OCC 2
#endif
constexpr float kTau = 8.f;   // the reference max moves only when a row max grows by more than
                              // this (log2 units): P stays <= 2^8 and most tiles skip the rescale

template <int D, int NW, int kBN>
__global__ void __launch_bounds__(NW * 64, CP_FWD_OCC) fwd_bf16_kernel(StepParams p) {
  constexpr int NT = NW * 64, BM = 32 * NW, KS = D / 16, NB = D / 32;
  constexpr int SB = kBN / 32;  // 32-key blocks per tile
  // LDS: region r holds K tile slot r followed by V tile slot 1 - r, so that the tiles one
  // iteration fills (K_{j+2}, V_{j+1}) form one region and the tiles it reads (K_{j+1}, V_j)
  // the other.
  constexpr int kTile = kBN * D;
  __shared__ __attribute__((aligned(16))) uint16_t sreg[2][2 * kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Work item: (kv head, query tile from the last one down, head within the group). Items of
  // one kv head are contiguous and map to one XCD, so its K/V stay in that XCD's L2; the
  // causally longest tiles start first.
  const int n_qt = (p.len_q + BM - 1) / BM;
  const int w = xcd_remap(blockIdx.x, n_qt * p.heads_q);
  const int h_in = w % p.group;
  const int rest = w / p.group;
  const int qt = n_qt - 1 - rest % n_qt;
  const int g = rest / n_qt;
  const int h = g * p.group + h_in;
  const int q_base = qt * BM;

  const uint16_t* qh = static_cast<const uint16_t*>(p.q) + (size_t)h * p.len_q * D;
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (size_t)g * p.len_kv * D;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + (size_t)g * p.len_kv * D;

  // This lane's query row, as the B operand of K Q^T: d = 16*ks + 8*half + t.
  const int qi = q_base + 32 * wave + col;
  const bool q_ok = qi < p.len_q;
  const int qi_c = q_ok ? qi : p.len_q - 1;
  u32x4_t qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4_t x = *reinterpret_cast<const u32x4_t*>(qh + (size_t)qi_c * D + 16 * ks + 8 * half);
    qreg[ks] = q_ok ? x : u32x4_t{0u, 0u, 0u, 0u};
  }

  // Keys any row of this workgroup may see.
  const int last_row = min(q_base + BM, p.len_q) - 1;
  long long nk = p.len_kv;
  if (p.causal) nk = min(nk, p.q_pos0 + last_row - p.kv_pos0 + 1);
  const int n_kt = nk > 0 ? (int)((nk + kBN - 1) / kBN) : 0;
  const int dpos = causal_shift(p.q_pos0, p.kv_pos0);
  const int wave_row0 = q_base + 32 * wave;

  using Dma = TileDma<D, kBN, NT>;

  f32x16_t oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x16_t{};
  float m_run = -INFINITY;  // reference row max of scale*log2(e)*s
  float l_run = 0.f;        // this lane's share of the running row sum

  const float c2 = p.scale_log2;

  // S^T = K Q^T of one tile from an LDS buffer; consecutive MFMAs go to different 32-key blocks
  // (independent accumulators).
  auto scores = [&](const uint16_t* kt_lds, f32x16_t (&sc)[SB]) {
#pragma unroll
    for (int blk = 0; blk < SB; ++blk) sc[blk] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int blk = 0; blk < SB; ++blk)
        sc[blk] = mfma32x32x16(tile_row8<D>(kt_lds, 32 * blk + perm_row(col), 2 * ks + half),
                               qreg[ks], sc[blk]);
  };

  // Software pipeline over key tiles, K one tile ahead of V. During iteration j the wave holds
  // S_j (computed in iteration j-1) and, while the VALU turns S_j into P_j, the matrix cores
  // compute S_{j+1}; then O += V_j^T P_j. LDS: K_{j+1} and V_j are resident; the direct loads of
  // K_{j+2} (into K_j's buffer) and V_{j+1} (into V_{j-1}'s) are in flight.
  f32x16_t s_a[SB], s_b[SB];  // S of the current tile and of the next one, alternating
  if (n_kt > 0) {
    Dma::issue(kg, 0, p.len_kv, sreg[0], wave, lane);           // K_0: K slot 0
    Dma::issue(vg, 0, p.len_kv, sreg[1] + kTile, wave, lane);   // V_0: V slot 0
    if (n_kt > 1) Dma::issue(kg, kBN, p.len_kv, sreg[1], wave, lane);  // K_1: K slot 1
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    scores(sreg[0], s_a);
    __syncthreads();  // every wave is done with K_0 before K_2 lands in its buffer
  }

  // One iteration. The region it fills by direct loads (wr: K_{j+2} into K slot j%2, V_{j+1}
  // into V slot (j+1)%2) and the region it reads (rd: K_{j+1}, V_j) are passed as restrict
  // pointers; knowing they are disjoint, the compiler does not make the LDS reads of V_j wait
  // for the loads in flight.
  auto iteration = [&](int kt, uint16_t* __restrict__ wr, const uint16_t* __restrict__ rd,
                       f32x16_t (&s_cur)[SB], f32x16_t (&s_nxt)[SB]) {
    uint16_t* const k_wr = wr;
    uint16_t* const v_wr = wr + kTile;
    const uint16_t* const k_rd = rd;
    const uint16_t* const v_rd = rd + kTile;
    if (kt + 1 < n_kt) Dma::issue(vg, (kt + 1) * kBN, p.len_kv, v_wr, wave, lane);
    if (kt + 2 < n_kt) Dma::issue(kg, (kt + 2) * kBN, p.len_kv, k_wr, wave, lane);
    const int key0 = kt * kBN;
    // every key of the tile visible to the wave's first row and inside the chunk?
    const bool full = key0 + kBN <= p.len_kv && (!p.causal || key0 + kBN - 1 - wave_row0 <= dpos);
    if (!full) {
#pragma unroll
      for (int blk = 0; blk < SB; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * blk + perm_row(8 * (r >> 2) + 4 * half + (r & 3));
          const bool vis = (key < p.len_kv) & ((!p.causal) | (key - qi <= dpos));
          s_cur[blk][r] = vis ? s_cur[blk][r] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < SB; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[blk][r]);
    mx = pair_max(mx) * c2;
    // Move the reference max only when the row max outgrew it by more than kTau (the first
    // visible tile always does: m_run starts at -inf). P = exp2(s*c2 - m_run) <= 2^kTau.
    const bool grow = mx > m_run + kTau;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
    m_run = grow ? mx : m_run;
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[nb][r] *= alpha;
    }

    // S_{j+1} on the matrix cores (independent of what follows) ... Unconditional so that it
    // shares a basic block with the exp work below; on the last tile it reads the other (stale
    // but in-bounds) K buffer and the result is discarded.
    scores(k_rd, s_nxt);
    // Let the scheduler interleave this block's LDS operand reads with the matrix products
    // (small-GEMM interleave strategy): 3.5% faster than its default schedule here.
    __builtin_amdgcn_iglp_opt(0);

    // ... while P_j = exp2(S_j*c2 - m) goes to bf16 (PV operand); the row sum stays fp32.
    u32x4_t pb[2 * SB];
    float lsum = 0.f;
#pragma unroll
    for (int blk = 0; blk < SB; ++blk)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[blk][8 * q + 2 * t], c2, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[blk][8 * q + 2 * t + 1], c2, -m_use));
          pb[2 * blk + q][t] = pack_bf16x2(p0, p1);
          lsum += p0 + p1;
        }
    l_run = l_run * alpha + lsum;

    // O^T += V^T P^T: the V^T operand for keys 16*kk .. 16*kk+15 via the transpose read.
#pragma unroll
    for (int kk = 0; kk < 2 * SB; ++kk)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        oacc[nb] = mfma32x32x16(tile_col8<D>(v_rd, 16 * kk, 32 * nb, lane), pb[kk], oacc[nb]);

  };
  // Unrolled by two so that the buffers and the S registers swap roles without copies.
  for (int kt = 0; kt < n_kt; kt += 2) {
    iteration(kt, sreg[0], sreg[1], s_a, s_b);
    // V_{j+1} and K_{j+2} have landed and every wave is done with V_j and K_{j+1}
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kt + 1 < n_kt) {
      iteration(kt + 1, sreg[1], sreg[0], s_b, s_a);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // Epilogue: O = O^T / l, LSE = ln(sum exp(s)) = (m + log2 l) * ln 2.
  const float l_tot = pair_sum(l_run);
  if (!q_ok) return;
  float inv, lse_new;
  if (l_tot > 0.f) {
    inv = 1.f / l_tot;
    lse_new = (m_run + log2f(l_tot)) * kLn2;
  } else {
    inv = 0.f;
    lse_new = -INFINITY;
  }
  float* orow = p.o + ((size_t)h * p.len_q + qi) * D;
  float* lrow = p.lse + (size_t)h * p.len_q + qi;
  if (!p.accumulate) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4_t v = {oacc[nb][4 * a4] * inv, oacc[nb][4 * a4 + 1] * inv,
                     oacc[nb][4 * a4 + 2] * inv, oacc[nb][4 * a4 + 3] * inv};
        *reinterpret_cast<f32x4_t*>(orow + 32 * nb + 8 * a4 + 4 * half) = v;
      }
    if (half == 0) *lrow = lse_new;
  } else if (lse_new != -INFINITY) {
    // Fold into the running (O, LSE): LSE' = logaddexp(old, new), weights exp(old - LSE') and
    // exp(new - LSE').
    const float lse_old = *lrow;
    const float hi = fmaxf(lse_old, lse_new);
    const float lse_m = hi + log1pf(expf(-fabsf(lse_old - lse_new)));
    const float wa = expf(lse_old - lse_m);
    const float wb = expf(lse_new - lse_m) * inv;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4_t* ptr = reinterpret_cast<f32x4_t*>(orow + 32 * nb + 8 * a4 + 4 * half);
        const f32x4_t old = *ptr;
        f32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = wa * old[e] + wb * oacc[nb][4 * a4 + e];
        *ptr = v;
      }
    if (half == 0) *lrow = lse_m;
  }
}

template <int D>
hipError_t launch_d(const StepParams& p, hipStream_t s) {
  constexpr int NW = CP_FWD_WAVES, BN = CP_FWD_KEYS;
  const int n_qt = (p.len_q + 32 * NW - 1) / (32 * NW);
  const dim3 grid((unsigned)(n_qt * p.heads_q));
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, BN>), grid, dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const StepParams& p, hipStream_t s) {
  if (p.head_dim == 128) return launch_d<128>(p, s);
  if (p.head_dim == 64) return launch_d<64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace cpa
