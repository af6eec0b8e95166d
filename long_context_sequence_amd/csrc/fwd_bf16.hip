// One ring step of the forward on gfx950: the rank's query tiles against one key/value chunk,
// bf16 MFMA for both contractions, online softmax in registers (StripedHyena 2
// context-parallelism page, section 2, ring attention steps 2-3).
//
// Work decomposition
//   workgroup = 8 wavefronts in two groups of 4: group A = waves 0-3, group B = waves 4-7.
//   Waves w and w + 4 share a SIMD. A group owns 128 query rows (32 per wave) of one head.
//   * pair workgroups: A and B take two heads of the same query tile (in a GQA group both read
//     the same key/value tiles, loaded once into LDS for both);
//   * split workgroups: A and B take the same 128 rows of one head and split its keys in two
//     halves; B hands its partial result to A through LDS at the end. A launch whose pair
//     workgroups would leave a last, partly filled round on the CUs turns those last pairs into
//     split workgroups of half the length (and so does a launch too small to fill the chip).
//
// Ping-pong schedule. Per 64-key tile j a wave runs two phases:
//   X_j: O^T += V_j^T P_j and S_{j+1}^T = K_{j+1} Q^T          (32 MFMAs, LDS operand reads)
//   Y_j: P_{j+1} = exp2(S_{j+1}^T * scale*log2e - m), running max/sum, O rescale  (VALU only)
// Group B runs one phase behind group A, and a workgroup barrier separates consecutive phases,
// so at any time one wave of each SIMD issues matrix products while the other does the softmax:
// the VALU work of one hides under the MFMAs of the other.
//
// Register-level formulation (per wave, per tile)
//   S^T[key][query] = K Q^T      A = K rows from LDS, B = the wave's Q rows held in registers
//   O^T[d][query] += V^T P^T     A = V^T rows from LDS (transpose read), B = P^T straight from
//                                the S^T accumulator registers (no LDS round trip for P)
// With S^T, each lane's accumulator column is one query row: the row max needs one swap with
// the lane 32 apart, the row sum stays lane-local until the end and the O rescale is one scalar
// per lane. Loading K row perm_row(m) for MFMA row m makes every run of 8 accumulator registers
// cover 8 consecutive keys, so the matching V^T operand is one transpose read (two
// ds_read_b64_tr_b16) of the row-major V tile.
//
// Causality: a group visits only tiles some of its rows can see; the mask is applied only on
// tiles that straddle the diagonal (for the wave's rows) or the ragged end of the chunk.
#include <math.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace cpa {
namespace {

constexpr int kBN = 64;       // keys per LDS tile
constexpr int kRows = 128;    // query rows per group (32 per wave)
// LDS operand reads in flight ahead of their product in the matrix phase; raised wave priority
// during that phase (the softmax wave on the same SIMD yields issue slots to it).
#ifndef CP_FWD_PF
#define CP_FWD_PF 4
#endif
#ifndef CP_FWD_PRIO
#define CP_FWD_PRIO 1
#endif
constexpr int kPF = CP_FWD_PF;
constexpr float kTau = 8.f;   // the reference max moves only when a row max grows by more than
                              // this (log2 units): P stays <= 2^8 and most tiles skip the rescale
// A tile whose P, against the current reference, sum to at most this has every P below 2^kTau
// (a rounded sum of non-negative terms is never below its largest term), so its row max cannot
// have outgrown the reference by more than kTau.
constexpr float kSumFast = 255.f;
static_assert(kTau == 8.f, "kSumFast must stay below 2^kTau");

// LDS of one group: K slots 0, 1 then V slots 0, 1, one 64 x D bf16 tile each.
template <int D>
constexpr int region_elems() { return 4 * kBN * D; }

// What one group of four waves computes: rows [q_base, q_base + 128) of head h against keys
// [key_lo, key_lo + 64 * n_tiles) of the chunk (its causal extent included).
struct GroupItem {
  int h;         // query head (-1: the group idles)
  int q_base;
  int key_lo;
  int n_tiles;
};

template <int D>
__global__ void __launch_bounds__(512, 1) fwd_bf16_kernel(StepParams p, int n_pair, int n_split) {
  constexpr int KS = D / 16, NB = D / 32;
  constexpr int SB = kBN / 32;  // 32-key blocks per tile
  constexpr int kTile = kBN * D;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * region_elems<D>()];

  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave_all >> 2;  // 0 = group A, 1 = group B
  const int wave = wave_all & 3;  // wave within the group

  const int n_qt = (p.len_q + kRows - 1) / kRows;
  // Keys any row of tile qt may see.
  auto key_count = [&](int qt) -> int {
    const int last_row = min((qt + 1) * kRows, p.len_q) - 1;
    long long nk = p.len_kv;
    if (p.causal) nk = min(nk, p.q_pos0 + last_row - p.kv_pos0 + 1);
    return nk > 0 ? (int)nk : 0;
  };
  // Pairs of heads: within a GQA group when its size is even (both heads then read the same
  // key/value head), else consecutive heads. Work order: pair within its block fastest, then
  // query tile from the last one down (causally longest first), then block; items of one
  // key/value head are contiguous and map to one XCD.
  const bool even_group = (p.group & 1) == 0;
  const int pairs_per_blk = even_group ? p.group / 2 : (p.heads_q + 1) / 2;
  const int blk_heads = even_group ? p.group : p.heads_q;
  auto pair_heads = [&](int w, int& h0, int& h1, int& qt) {
    const int p_in = w % pairs_per_blk;
    const int rest = w / pairs_per_blk;
    qt = n_qt - 1 - rest % n_qt;
    const int blk = rest / n_qt;
    h0 = blk * blk_heads + 2 * p_in;
    h1 = h0 + 1 < p.heads_q ? h0 + 1 : -1;
  };

  GroupItem it;
  bool split = false;   // both groups on one head, keys split in two halves
  bool shared = false;  // both groups read the same key/value tiles (loaded by group A)
  int n_loop;           // tiles both groups step through (the longer group's count)
  if ((int)blockIdx.x < n_pair) {
    int h0, h1, qt;
    pair_heads(xcd_remap(blockIdx.x, n_pair), h0, h1, qt);
    it.h = grp == 0 ? h0 : h1;
    it.q_base = qt * kRows;
    it.key_lo = 0;
    it.n_tiles = (key_count(qt) + kBN - 1) / kBN;
    n_loop = it.n_tiles;  // same query tile for both groups: same extent
    shared = h1 >= 0 && h0 / p.group == h1 / p.group;
  } else {
    const int s = xcd_remap(blockIdx.x - n_pair, n_split);
    int h0, h1, qt;
    pair_heads(n_pair + s / 2, h0, h1, qt);
    const int h = (s & 1) ? h1 : h0;
    if (h < 0) return;  // the whole workgroup idles (odd head count)
    split = true;
    const int nt = (key_count(qt) + kBN - 1) / kBN;
    const int n_a = (nt + 1) / 2;
    it.h = h;
    it.q_base = qt * kRows;
    it.key_lo = grp == 0 ? 0 : n_a * kBN;
    it.n_tiles = grp == 0 ? n_a : nt - n_a;
    n_loop = n_a;
  }
  const bool active = it.h >= 0;
  const int g = active ? it.h / p.group : 0;
  // LDS slots. Separate tiles: each group has its own region of two K and two V slots. Shared
  // tiles: one region of three K and three V slots; group A loads the K tiles, group B the V
  // tiles, so that both groups carry half of the load issue.
  uint16_t* const my_lds = lds + grp * region_elems<D>();
  auto KSLOT = [&](int s) { return my_lds + s * kTile; };
  auto VSLOT = [&](int s) { return my_lds + (2 + s) * kTile; };
  auto KSH = [&](int s) { return lds + s * kTile; };
  auto VSH = [&](int s) { return lds + (3 + s) * kTile; };
  static_assert(6 * kTile <= 2 * region_elems<D>(), "three shared K and V slots fit");

  const uint16_t* qh = static_cast<const uint16_t*>(p.q) + (size_t)(active ? it.h : 0) * p.len_q * D;
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (size_t)g * p.len_kv * D;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + (size_t)g * p.len_kv * D;

  // This lane's query row, as the B operand of K Q^T: d = 16*ks + 8*half + t.
  const int qi = it.q_base + 32 * wave + col;
  const bool q_ok = active && qi < p.len_q;
  const int qi_c = q_ok ? qi : 0;
  u32x4_t qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4_t x = *reinterpret_cast<const u32x4_t*>(qh + (size_t)qi_c * D + 16 * ks + 8 * half);
    qreg[ks] = q_ok ? x : u32x4_t{0u, 0u, 0u, 0u};
  }
  const int dpos = causal_shift(p.q_pos0, p.kv_pos0);
  const int wave_row0 = it.q_base + 32 * wave;
  const int n_own = active ? it.n_tiles : 0;

  // The running (O, LSE) that the epilogue folds this step into, fetched before the last tile's
  // products so that the loads overlap them (only the lanes that fold: group B of a split
  // workgroup hands its partial to group A instead).
  f32x4_t o_old[4 * NB];
  float lse_old = -INFINITY;
  const bool folds = p.accumulate && q_ok && n_own > 0 && !(split && grp == 1);
  auto fetch_old = [&]() __attribute__((always_inline)) {
    if (!folds) return;
    const float* orow = p.o + ((size_t)it.h * p.len_q + qi) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
        o_old[4 * nb + a4] = *reinterpret_cast<const f32x4_t*>(orow + 32 * nb + 8 * a4 + 4 * half);
    lse_old = p.lse[(size_t)it.h * p.len_q + qi];
  };

  using Dma = TileDma<D, kBN, 256>;
  // Direct loads of tile t (keys key_lo + 64 t ...) of K or V into a slot.
  auto load_k = [&](int t, uint16_t* slot) __attribute__((always_inline)) {
    Dma::issue(kg, it.key_lo + t * kBN, p.len_kv, slot, wave, lane);
  };
  auto load_v = [&](int t, uint16_t* slot) __attribute__((always_inline)) {
    Dma::issue(vg, it.key_lo + t * kBN, p.len_kv, slot, wave, lane);
  };

  f32x16_t oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x16_t{};
  float m_run = -INFINITY;  // reference row max of scale*log2(e)*s
  float l_run = 0.f;        // this lane's share of the running row sum
  const float c2 = p.scale_log2;
  f32x16_t sc[SB];   // S^T of the next tile
  u32x4_t pb[2 * SB];  // P^T of the current tile, bf16 pairs (the PV operand)

  // Phase X_j: O^T += V_j^T P_j (j >= 0), S_{j+1}^T = K_{j+1} Q^T. The products' LDS operands
  // are read kPF products ahead of their use, with scheduling fences keeping that order: one
  // wavefront per SIMD issues products in this phase, so nothing else hides the LDS latency.
  // PV product i: 16-key step i / NB, d block i % NB; S product i: d step i / SB, 32-key block
  // i % SB.
  auto pv_load = [&](const uint16_t* v_rd, int i) {
    return tile_col8<D>(v_rd, 16 * (i / NB), 32 * (i % NB), lane);
  };
  auto s_load = [&](const uint16_t* k_rd, int i) {
    return tile_row8<D>(k_rd, 32 * (i % SB) + perm_row(col), 2 * (i / SB) + half);
  };
  auto pv_step = [&](int i, const u32x4_t& a) {
    oacc[i % NB] = mfma32x32x16(a, pb[i / NB], oacc[i % NB]);
  };
  auto s_step = [&](int i, const u32x4_t& a) {
    sc[i % SB] = mfma32x32x16(a, qreg[i / SB], sc[i % SB]);
  };
  constexpr int NPV = 2 * SB * NB, NS = KS * SB;
  constexpr int kMove = NB;  // PV products of the tile's last 16-key step (one per d block)
  auto zero_s = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int blk = 0; blk < SB; ++blk) sc[blk] = f32x16_t{};
  };
  // X_j inside the loop: both products. On a group's last tile S is computed from the other K
  // slot (stale but in-bounds) and discarded; the last phase of the loop is peeled instead.
  auto phase_x = [&](const uint16_t* __restrict__ v_rd, const uint16_t* __restrict__ k_rd) __attribute__((always_inline)) {
    zero_s();
    if (CP_FWD_PRIO) __builtin_amdgcn_s_setprio(1);
    // Products in groups of seven, S PV S PV S PV S: S has two accumulators, and a product must
    // not follow the product that accumulates into the same registers too closely. The PV
    // products of the tile's last 16-key step run at the start of Y_j instead (pv_tail), which
    // balances the two phases.
    static_assert(NPV == NS && NS % 4 == 0, "groups of four S and three PV products");
    mfma_seq<NS + NPV - kMove, kPF>(
        [&](int i) {
          const int g7 = i / 7, r7 = i % 7;
          return (r7 & 1) == 0 ? s_load(k_rd, 4 * g7 + r7 / 2) : pv_load(v_rd, 3 * g7 + r7 / 2);
        },
        [&](int i, const u32x4_t& a) {
          const int g7 = i / 7, r7 = i % 7;
          if ((r7 & 1) == 0) s_step(4 * g7 + r7 / 2, a);
          else pv_step(3 * g7 + r7 / 2, a);
        });
    if (CP_FWD_PRIO) __builtin_amdgcn_s_setprio(0);
  };
  // The PV products X_j left out: O^T += V_j^T P_j over the tile's last 16 keys (before Y_j
  // overwrites those P).
  auto pv_tail = [&](const uint16_t* __restrict__ v_rd) __attribute__((always_inline)) {
    mfma_seq<kMove, 2>([&](int i) { return pv_load(v_rd, NPV - kMove + i); },
                           [&](int i, const u32x4_t& a) { pv_step(NPV - kMove + i, a); });
  };
  // Phase Y_j: softmax of S_{j+1}: mask, running max (lazy rescale of O and the sum), P to bf16.
  auto phase_y = [&](int j) __attribute__((always_inline)) {
    if (j + 1 >= n_own) return;
    const int key0 = it.key_lo + (j + 1) * kBN;
    // every key of the tile visible to the wave's first row and inside the chunk?
    const bool full = key0 + kBN <= p.len_kv && (!p.causal || key0 + kBN - 1 - wave_row0 <= dpos);
    if (!full) {
#pragma unroll
      for (int blk = 0; blk < SB; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * blk + perm_row(8 * (r >> 2) + 4 * half + (r & 3));
          const bool vis = (key < p.len_kv) & ((!p.causal) | (key - qi <= dpos));
          sc[blk][r] = vis ? sc[blk][r] : -INFINITY;
        }
    }
    // P = exp2(s*c2 - m) against reference max m, packed to bf16 pairs; returns the row sum.
    auto exps = [&](float m_use) __attribute__((always_inline)) -> float {
      float ls = 0.f;
#pragma unroll
      for (int blk = 0; blk < SB; ++blk)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[blk][8 * q + 2 * t], c2, -m_use));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[blk][8 * q + 2 * t + 1], c2, -m_use));
            pb[2 * blk + q][t] = pack_bf16x2(p0, p1);
            ls += p0 + p1;
          }
      return ls;
    };
    // First against the current reference max. A lane's sum (its half of the row's 64 P) of at
    // most kSumFast bounds every P it holds below 2^kTau; when that holds in every lane the
    // reference stays, exactly as the row-max test below would decide, and the row max is never
    // needed. A larger sum, or inf / NaN (no reference yet: m_run = -inf), in any lane sends the
    // wave through that test.
    float alpha = 1.f;
    float lsum = exps(m_run);
    if (__builtin_amdgcn_ballot_w64(!(lsum <= kSumFast)) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < SB; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[blk][r]);
      mx = pair_max(mx) * c2;
      // Move the reference max only when the row max outgrew it by more than kTau (the first
      // visible tile always does: m_run starts at -inf). P = exp2(s*c2 - m_run) <= 2^kTau.
      const bool grow = mx > m_run + kTau;
      alpha = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
      m_run = grow ? mx : m_run;
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[nb][r] *= alpha;
      }
      lsum = exps(m_use);
    }
    l_run = l_run * alpha + lsum;
  };
  // Workgroup barrier between phases; the scheduling fences keep each phase's instructions on
  // its own side.
  auto bar = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  // X of a last tile: PV alone.
  auto phase_x_last = [&](const uint16_t* v_rd) __attribute__((always_inline)) {
    if (CP_FWD_PRIO) __builtin_amdgcn_s_setprio(1);
    mfma_seq<NPV, kPF>([&](int i) { return pv_load(v_rd, i); }, pv_step);
    if (CP_FWD_PRIO) __builtin_amdgcn_s_setprio(0);
  };
  auto phase_s0 = [&](const uint16_t* k_rd) __attribute__((always_inline)) {  // X_{-1}: S_0 alone
    zero_s();
    mfma_seq<NS, kPF>([&](int i) { return s_load(k_rd, i); }, s_step);
  };
  // Tile j: X_j reads V_j and K_{j+1}; Y_j turns S_{j+1} into P_{j+1}. The loops below are
  // unrolled by the slot count so that slots are compile-time constants; the last tile (PV
  // alone) follows each loop.
  const int n_body = n_loop - 1;
  if (shared) {
    // Both groups step through the same n tiles, group B one phase behind group A. Tile t sits
    // in slot t % 3, and each group issues its loads at the start of its X phase, where the
    // matrix products leave issue slots free: A issues K_{j+3} in X_j (into K_j's slot: both
    // groups read K_j in X_{j-1}), B issues V_{j+2} in X_j (into V_{j-1}'s slot: both groups
    // have read V_{j-1} by then). A waits for K_{j+2} at the end of its Y_j, B for V_{j+1} at the
    // end of its X_j, each just before the barrier ahead of the first reader's X; the wait lets
    // the group's newer load stay in flight.
    const int n = n_loop;
    if (grp == 0) {
      if (n > 0) load_k(0, KSH(0));
      if (n > 1) load_k(1, KSH(1));
    } else {
      if (n > 0) load_v(0, VSH(0));
    }
    __builtin_amdgcn_s_waitcnt(0);
    bar();
    if (grp == 1) bar();  // group B runs one phase behind
    if (grp == 0 && 2 < n) load_k(2, KSH(2));
    if (grp == 1 && 1 < n) load_v(1, VSH(1));
    if (n > 0) phase_s0(KSH(0));
    bar();
    phase_y(-1);
    auto tile = [&](int j, int s) __attribute__((always_inline)) {  // s = j % 3
      bar();
      if (grp == 0 && j + 3 < n) load_k(j + 3, KSH(s));
      if (grp == 1 && j + 2 < n) load_v(j + 2, VSH(s == 0 ? 2 : s - 1));
      phase_x(VSH(s), KSH(s == 2 ? 0 : s + 1));
      if (grp == 1) {  // V_{j+1} complete; V_{j+2} may stay in flight
        if (j + 2 < n) wait_vmcnt<Dma::ITERS>();
        else wait_vmcnt<0>();
      }
      bar();
      pv_tail(VSH(s));
      phase_y(j);
      if (grp == 0) {  // K_{j+2} complete; K_{j+3} may stay in flight
        if (j + 3 < n) wait_vmcnt<Dma::ITERS>();
        else wait_vmcnt<0>();
      }
    };
    for (int j = 0; j < n_body; j += 3) {
      tile(j, 0);
      if (j + 1 < n_body) {
        tile(j + 1, 1);
        if (j + 2 < n_body) tile(j + 2, 2);
      }
    }
    if (n > 0) {
      fetch_old();
      bar();
      phase_x_last(VSH((n - 1) % 3));
      bar();
    }
  } else {
    // Each group loads its own tiles into its own region, two slots each. K_{j+2} (into K_j's
    // slot) and V_{j+1} (into V_{j-1}'s slot) are issued at the start of X_j and waited for at
    // the end of Y_j. In a split workgroup group B may have one tile fewer than group A; it
    // then idles through A's last phase pair.
    if (n_own > 0) {
      load_k(0, KSLOT(0));
      if (n_own > 1) load_k(1, KSLOT(1));
      load_v(0, VSLOT(0));
    }
    __builtin_amdgcn_s_waitcnt(0);
    bar();
    if (grp == 1) bar();  // group B runs one phase behind
    if (n_own > 0) phase_s0(KSLOT(0));
    bar();
    phase_y(-1);
    auto tile = [&](int j, int s) __attribute__((always_inline)) {  // s = j % 2
      bar();
      if (j + 2 < n_own) load_k(j + 2, KSLOT(s));
      if (j + 1 < n_own) load_v(j + 1, VSLOT(1 - s));
      if (j < n_own) phase_x(VSLOT(s), KSLOT(1 - s));
      bar();
      if (j < n_own) pv_tail(VSLOT(s));
      phase_y(j);
      __builtin_amdgcn_s_waitcnt(0);
    };
    for (int j = 0; j < n_body; j += 2) {
      tile(j, 0);
      if (j + 1 < n_body) tile(j + 1, 1);
    }
    if (n_loop > 0) {
      const int j = n_loop - 1;
      fetch_old();
      bar();
      if (j < n_own) phase_x_last(VSLOT(j & 1));
      bar();
    }
  }
  if (grp == 0) bar();  // group A ends one phase earlier

  if (split) {
    // B's partial (O^T, running max, its lanes' sums) goes through LDS to A, which folds it into
    // its own: both are scaled to the larger reference max. The tiles are no longer read.
    float* const xch = reinterpret_cast<float*>(lds) + wave * (NB * 16 + 2) * 64;
    if (grp == 1) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[(16 * nb + r) * 64 + lane] = oacc[nb][r];
      xch[(16 * NB) * 64 + lane] = m_run;
      xch[(16 * NB + 1) * 64 + lane] = l_run;
    }
    bar();
    if (grp == 1) return;
    const float m_b = xch[(16 * NB) * 64 + lane];
    const float l_b = xch[(16 * NB + 1) * 64 + lane];
    const float m_new = fmaxf(m_run, m_b);
    const float wa = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float wb = m_b == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_b - m_new);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[nb][r] = wa * oacc[nb][r] + wb * xch[(16 * nb + r) * 64 + lane];
    l_run = wa * l_run + wb * l_b;
    m_run = m_new;
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
  float* orow = p.o + ((size_t)it.h * p.len_q + qi) * D;
  float* lrow = p.lse + (size_t)it.h * p.len_q + qi;
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
    const float hi = fmaxf(lse_old, lse_new);
    const float lse_m = hi + log1pf(expf(-fabsf(lse_old - lse_new)));
    const float wa = expf(lse_old - lse_m);
    const float wb = expf(lse_new - lse_m) * inv;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4_t* ptr = reinterpret_cast<f32x4_t*>(orow + 32 * nb + 8 * a4 + 4 * half);
        const f32x4_t old = o_old[4 * nb + a4];
        f32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = wa * old[e] + wb * oacc[nb][4 * a4 + e];
        *ptr = v;
      }
    if (half == 0) *lrow = lse_m;
  }
}

}  // namespace

int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev] = n;
  return n;
}

namespace {

template <int D>
hipError_t launch_d(const StepParams& p, hipStream_t s) {
  const int n_qt = (p.len_q + kRows - 1) / kRows;
  const long long n_pairs = (long long)n_qt * ((p.group & 1) == 0 ? p.heads_q / 2
                                                                   : (p.heads_q + 1) / 2);
  // One workgroup per CU at a time. When every pair has the same work (every key visible to
  // every row) and the last round of pair workgroups would fill at most half of the CUs, its
  // pairs run as split workgroups instead: two per pair, each of half the length, so the last
  // round takes half the time. A launch with fewer pairs than half the CUs is split in full. A
  // causal step with masking is left whole: its pairs differ in length, the longest run first
  // and the short ones fill the end.
  const int cus = device_cus();
  const bool uniform = !p.causal || p.kv_pos0 + p.len_kv - 1 <= p.q_pos0;
  const long long rem = n_pairs % cus;
  const bool split_tail = rem > 0 && 2 * rem <= cus && (uniform || n_pairs < cus);
  const long long n_split_pairs = split_tail ? rem : 0;
  const int n_pair = (int)(n_pairs - n_split_pairs);
  const int n_split = (int)(2 * n_split_pairs);
  if (n_pair + n_split == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_bf16_kernel<D>), dim3((unsigned)(n_pair + n_split)), dim3(512), 0, s,
                     p, n_pair, n_split);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const StepParams& p, hipStream_t s) {
  if (p.head_dim == 128) return launch_d<128>(p, s);
  if (p.head_dim == 64) return launch_d<64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace cpa
