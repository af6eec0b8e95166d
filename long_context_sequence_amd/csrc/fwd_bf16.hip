// One ring step of the forward on gfx950: the rank's query tile against one key/value chunk,
// bf16 MFMA for both contractions, online softmax in registers (StripedHyena 2
// context-parallelism page, section 2, ring attention steps 2-3).
//
// Work decomposition
//   workgroup = NW waves = one query head x BM = 32*NW query rows; each wave owns 32 rows.
//   Keys stream through LDS in tiles of 64 (double buffered): K row-major, V transposed.
//
// Register-level formulation (per wave, per 64-key tile)
//   S^T[key][query] = K Q^T      A = K rows from LDS, B = the wave's Q rows held in registers
//   P^T = exp2(S^T * scale*log2e - m)
//   O^T[d][query] += V^T P^T     A = V^T rows from LDS, B = P^T straight from the S^T
//                                accumulator registers (no LDS round trip for P)
// With S^T, each lane's accumulator column is one query row, so the row max needs one swap with
// the lane 32 apart, the row sum stays lane-local until the end and the O rescale is one scalar
// per lane. Loading K row perm_row(m) for MFMA row m makes every run of 8 accumulator registers
// cover 8 consecutive keys, so the matching V^T operand is one 16-byte LDS read.
//
// Causality: a tile is computed only if some key in it is visible to some row of the wave;
// the mask is applied only on tiles that straddle the diagonal or the ragged end of the chunk.
#include <math.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace cpa {
namespace {

constexpr int kBN = 64;  // keys per tile

template <int D, int NW>
struct FwdShape {
  static constexpr int NT = NW * 64;            // threads
  static constexpr int BM = 32 * NW;            // query rows per workgroup
  static constexpr int KCH = D / 8;             // 16-byte chunks per K row
  static constexpr int KS = D / 16;             // k-steps of Q K^T
  static constexpr int NB = D / 32;             // 32-row blocks of O^T
  static constexpr int KLD = kBN * KCH / NT;    // K chunks staged per thread
  static constexpr int VUNITS = (kBN / 8) * (D / 4);  // V pieces of 8 keys x 4 columns
  static constexpr int VLD = (VUNITS + NT - 1) / NT;
  static_assert(kBN * KCH % NT == 0, "K tile must split evenly over the threads");
};

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64, 2) fwd_bf16_kernel(StepParams p) {
  using S = FwdShape<D, NW>;
  constexpr int NT = S::NT, BM = S::BM, KCH = S::KCH, KS = S::KS, NB = S::NB;
  __shared__ __attribute__((aligned(16))) uint16_t sk[2][kBN * D];
  __shared__ __attribute__((aligned(16))) uint16_t svt[2][D * kBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;

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

  u32x4_t kst[S::KLD];
  u32x2_t vst[S::VLD][8];

  auto load_tile = [&](int kt) {
    const int key0 = kt * kBN;
#pragma unroll
    for (int u = 0; u < S::KLD; ++u) {
      const int idx = tid + u * NT;
      const int r = idx / KCH, c = idx % KCH;
      const int key = key0 + r;
      const bool ok = key < p.len_kv;
      const int kc = ok ? key : p.len_kv - 1;
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(kg + (size_t)kc * D + 8 * c);
      kst[u] = ok ? x : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < S::VLD; ++u) {
      const int unit = tid + u * NT;
      if (unit < S::VUNITS) {
        const int cg = unit % (D / 4), rg = unit / (D / 4);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int key = key0 + 8 * rg + r;
          const bool ok = key < p.len_kv;
          const int kc = ok ? key : p.len_kv - 1;
          u32x2_t x = *reinterpret_cast<const u32x2_t*>(vg + (size_t)kc * D + 4 * cg);
          vst[u][r] = ok ? x : u32x2_t{0u, 0u};
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < S::KLD; ++u) {
      const int idx = tid + u * NT;
      const int r = idx / KCH, c = idx % KCH;
      const int pos = c ^ swz_rows<KCH>(r);
      *reinterpret_cast<u32x4_t*>(&sk[buf][r * D + 8 * pos]) = kst[u];
    }
#pragma unroll
    for (int u = 0; u < S::VLD; ++u) {
      const int unit = tid + u * NT;
      if (unit < S::VUNITS) {
        const int cg = unit % (D / 4), rg = unit / (D / 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          // column n = 4*cg + c of keys 8*rg .. 8*rg+7, packed two keys per word
          const int n = 4 * cg + c;
          const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
          u32x4_t out;
#pragma unroll
          for (int pq = 0; pq < 4; ++pq)
            out[pq] = __builtin_amdgcn_perm(vst[u][2 * pq + 1][c >> 1], vst[u][2 * pq][c >> 1], sel);
          const int pos = rg ^ swz_t(n);
          *reinterpret_cast<u32x4_t*>(&svt[buf][n * kBN + 8 * pos]) = out;
        }
      }
    }
  };

  f32x16_t oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x16_t{};
  float m_run = -INFINITY;  // running row max of scale*log2(e)*s
  float l_run = 0.f;        // this lane's share of the running row sum

  if (n_kt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  const long long wave_q0 = p.q_pos0 + q_base + 32 * wave;  // global position of the wave's row 0
  const float c2 = p.scale_log2;

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) load_tile(kt + 1);
    const long long key_pos0 = p.kv_pos0 + (long long)kt * kBN;
    const bool wave_visible = !p.causal || key_pos0 <= wave_q0 + 31;
    if (wave_visible) {
      f32x16_t s[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        s[blk] = f32x16_t{};
        const int row = 32 * blk + perm_row(col);
        const int sw = swz_rows<KCH>(row);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int pos = (2 * ks + half) ^ sw;
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&sk[buf][row * D + 8 * pos]);
          s[blk] = mfma32x32x16(a, qreg[ks], s[blk]);
        }
      }
      const bool need_mask =
          (kt * kBN + kBN > p.len_kv) || (p.causal && key_pos0 + kBN - 1 > wave_q0);
      if (need_mask) {
        const long long qpos = wave_q0 + col;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt * kBN + 32 * blk + perm_row(8 * (r >> 2) + 4 * half + (r & 3));
            const bool vis = key < p.len_kv && (!p.causal || p.kv_pos0 + key <= qpos);
            if (!vis) s[blk][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[blk][r]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx * c2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;

      u32x4_t pb[4];
      float lsum = 0.f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[blk][8 * q + 2 * t], c2, -m_use));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[blk][8 * q + 2 * t + 1], c2, -m_use));
            lsum += p0 + p1;
            pb[2 * blk + q][t] = pack_bf16x2(p0, p1);
          }
      l_run = l_run * alpha + lsum;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[nb][r] *= alpha;
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int n = 32 * nb + col;
        const int sw = swz_t(n);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int pos = (2 * kk + half) ^ sw;
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&svt[buf][n * kBN + 8 * pos]);
          oacc[nb] = mfma32x32x16(a, pb[kk], oacc[nb]);
        }
      }
    }
    if (kt + 1 < n_kt) store_tile(buf ^ 1);
    __syncthreads();
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
  constexpr int NW = 4;
  const int n_qt = (p.len_q + 32 * NW - 1) / (32 * NW);
  const dim3 grid((unsigned)(n_qt * p.heads_q));
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW>), grid, dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const StepParams& p, hipStream_t s) {
  if (p.head_dim == 128) return launch_d<128>(p, s);
  if (p.head_dim == 64) return launch_d<64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace cpa
