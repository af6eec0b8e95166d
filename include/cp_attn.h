/*
 * cp_attn — one context-parallel rank's ring-attention work on an AMD MI355X (gfx950).
 *
 * The method (StripedHyena 2 context-parallelism page, section 2, "ring attention: passing
 * key/value around the ring", steps 1-4): the sequence of L tokens is cut into N_cp contiguous
 * chunks (section 1 of the same page: shards of [D, L/N_cp]). A rank keeps its query shard, and
 * at each ring step attends to the one key/value chunk it currently holds, folding the partial
 * result into a running output with online-softmax statistics. After N_cp steps it holds its
 * shard of full attention. Under causal masking (section 5 of that page: causal work is
 * triangular) chunks after the rank's own need no work. Grouped-query attention (2D-attention
 * summary, "LLM architecture" section; Ulysses explainer, ring-vs-Ulysses section) lets a group
 * of query heads share one key/value head.
 *
 * Conventions shared by every call
 *  - Memory: every tensor pointer is device memory (hipMalloc or torch), 16-byte aligned,
 *    row-major and contiguous. Q, dO: [heads_q, len_q, head_dim]. K, V: [heads_kv, len_kv,
 *    head_dim]. O, dQ: [heads_q, len_q, head_dim] fp32. dK, dV: [heads_kv, len_kv, head_dim]
 *    fp32. LSE, delta: [heads_q, len_q] fp32. head_dim is innermost.
 *  - Heads: query head h reads key/value head h / (heads_q / heads_kv) (contiguous groups).
 *  - Positions: row i of Q sits at global position q_pos0 + i, row j of K/V at kv_pos0 + j.
 *    For contiguous chunks of length Lc, chunk c starts at c * Lc. Causal: the query at
 *    position p sees keys at positions <= p (itself included).
 *  - Scale: scores are scale * (q . k); scale <= 0 selects 1/sqrt(head_dim).
 *  - LSE is the natural-log log-sum-exp of the scaled scores over the visible keys; a row that
 *    sees no key has O = 0 and LSE = -inf.
 *  - Ownership: the caller allocates and frees everything; the library allocates nothing,
 *    keeps no pointer after a call returns and holds no mutable global state.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls only
 *    enqueue work; CP_OK means "enqueued". Calls on different streams may run concurrently if
 *    their outputs do not overlap.
 *  - Errors: arguments are validated before anything is enqueued; on any error nothing is
 *    written. CP_ERR_HIP reports a failed launch. No C++ exception crosses this boundary.
 *    NaN/Inf inputs are not checked and propagate.
 *  - Supported: head_dim 64 or 128; dtype CP_BF16 for every call, CP_F32 for cp_attn_step
 *    (the fp32 path is a plain VALU kernel meant for small, accuracy-critical cases) and
 *    cp_attn_bwd_prep. Lengths up to CP_MAX_LEN, heads up to CP_MAX_HEADS.
 */
#ifndef CP_ATTN_H
#define CP_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CP_MAX_LEN (1 << 23)   /* rows per shard/chunk: keeps per-head byte offsets < 4 GB */
#define CP_MAX_HEADS 1024

typedef enum {
  CP_OK = 0,
  CP_STEP_SKIPPED = 1,      /* causal and every key is after every query: nothing enqueued */
  CP_ERR_NULL = -1,         /* a required pointer is NULL */
  CP_ERR_SHAPE = -2,        /* sizes out of range or inconsistent */
  CP_ERR_DTYPE = -3,        /* unknown dtype */
  CP_ERR_ALIGN = -4,        /* a pointer is not 16-byte aligned */
  CP_ERR_UNSUPPORTED = -5,  /* valid request this build does not implement (e.g. head_dim 96) */
  CP_ERR_HIP = -6,          /* the HIP runtime reported an error at launch */
  CP_ERR_SCRATCH_LIMIT = -7 /* larger than the fixed scratch of an allocation-free entry point */
} cp_status;

typedef enum { CP_F32 = 0, CP_BF16 = 1 } cp_dtype;

/* One ring step: the rank's queries against one key/value chunk. Positions are explicit
 * (q_pos0, kv_pos0) rather than chunk indices, so that contiguous, zig-zag and striped
 * placements all use the same call: for contiguous chunks of length Lc, chunk c starts at
 * c * Lc. `accumulate` lets a step fold into the running (O, LSE) without a separate merge. */
typedef struct {
  int32_t heads_q;     /* query heads; a multiple of heads_kv */
  int32_t heads_kv;    /* key/value heads */
  int32_t len_q;       /* query rows of the shard (>= 0) */
  int32_t len_kv;      /* key/value rows of the chunk (>= 0) */
  int32_t head_dim;    /* 64 or 128 */
  int32_t causal;      /* 0 or 1 */
  int64_t q_pos0;      /* global position of query row 0 */
  int64_t kv_pos0;     /* global position of key/value row 0 */
  float scale;         /* <= 0: 1/sqrt(head_dim) */
  int32_t dtype;       /* cp_dtype of q, k, v (and d_o for the backward) */
  int32_t accumulate;  /* cp_attn_step only: 0 = write this step's (O, LSE);
                          1 = fold this step into the running (O, LSE) already in o/lse */
} cp_attn_desc;

/*
 * cp_attn_step — partial attention of the rank's queries against the chunk it holds, with the
 * online-softmax statistics of that step (context-parallelism page, section 2, ring attention
 * steps 2-3). Keys causally invisible to a whole tile are skipped, not computed.
 *   q   [heads_q, len_q, head_dim] (dtype)
 *   k,v [heads_kv, len_kv, head_dim] (dtype)
 *   o   [heads_q, len_q, head_dim] fp32, normalised output of this step (accumulate = 0) or the
 *       running output updated in place (accumulate = 1)
 *   lse [heads_q, len_q] fp32, natural-log LSE of this step / running LSE updated in place
 * accumulate = 1 equals cp_attn_step into scratch followed by cp_attn_merge, in one pass.
 * Returns CP_STEP_SKIPPED (nothing enqueued, nothing written) when causal and no key is
 * visible to any query. A row that sees no key gets (0, -inf) with accumulate = 0 and is left
 * unchanged with accumulate = 1.
 */
cp_status cp_attn_step(const cp_attn_desc* desc, const void* q, const void* k, const void* v,
                       float* o, float* lse, void* stream);

/*
 * cp_attn_merge — fold one step's partial result into the running one (online softmax over
 * disjoint key sets; context-parallelism page, section 2, ring attention step 3):
 *   LSE' = log(exp(lse_acc) + exp(lse)),
 *   o_acc' = exp(lse_acc - LSE') * o_acc + exp(lse - LSE') * o,   both in place.
 * rows = heads_q * len_q. Two empty rows (-inf, -inf) give (0, -inf).
 *   o_acc, o [rows, head_dim] fp32; lse_acc, lse [rows] fp32. o/lse are read only.
 */
cp_status cp_attn_merge(int64_t rows, int32_t head_dim, float* o_acc, float* lse_acc,
                        const float* o, const float* lse, void* stream);

/*
 * cp_attn_bwd_prep — delta[r] = sum_t dO[r, t] * O[r, t] per row (rows = heads_q * len_q), the
 * softmax-Jacobian term the backward needs (since O_i = sum_j P_ij V_j, it equals
 * sum_j P_ij (dO_i . V_j)). O is the final fp32 forward output; d_o has `dtype` (CP_BF16 or
 * CP_F32), the same [rows, head_dim] layout. delta: [rows] fp32, overwritten.
 * The pages describe only the forward ring; the backward calls here are the gradient of that
 * forward (loss = sum(O * dO)) through the softmax Jacobian, with P recomputed from the saved
 * LSE instead of being stored.
 */
cp_status cp_attn_bwd_prep(int64_t rows, int32_t head_dim, int32_t dtype, const float* o,
                           const void* d_o, float* delta, void* stream);

/*
 * cp_attn_bwd — one ring step of the backward (dtype CP_BF16): the gradient of
 * loss = sum(O * dO) restricted to this chunk's keys (the gradient of cp_attn_step's forward;
 * the pages give no backward), recomputing P = exp(S - LSE) from the final forward LSE instead
 * of storing it:
 *   dV_c += P^T dO,  dP = dO V_c^T,  dS = P * (dP - delta),
 *   dQ += scale * dS K_c,  dK_c += scale * dS^T Q   (dK, dV summed over each head group).
 *   d_o [heads_q, len_q, head_dim] (dtype); lse, delta [heads_q, len_q] fp32 (final forward
 *   LSE and cp_attn_bwd_prep's output); dq [heads_q, len_q, head_dim] fp32;
 *   dk, dv [heads_kv, len_kv, head_dim] fp32. dq, dk, dv are accumulated (+=): zero them
 *   before the first step. desc->accumulate is ignored.
 * Returns CP_STEP_SKIPPED when causal and no key is visible to any query.
 */
cp_status cp_attn_bwd(const cp_attn_desc* desc, const void* q, const void* k, const void* v,
                      const void* d_o, const float* lse, const float* delta, float* dq,
                      float* dk, float* dv, void* stream);

/*
 * cp_attn_bwd_dkdv / cp_attn_bwd_dq — the two halves of cp_attn_bwd, one kernel each, same
 * arguments and semantics: the first accumulates dk and dv only (dq is not touched and may be
 * NULL), the second accumulates dq only (dk, dv may be NULL). cp_attn_bwd = both, in this order.
 */
cp_status cp_attn_bwd_dkdv(const cp_attn_desc* desc, const void* q, const void* k,
                           const void* v, const void* d_o, const float* lse,
                           const float* delta, float* dk, float* dv, void* stream);
cp_status cp_attn_bwd_dq(const cp_attn_desc* desc, const void* q, const void* k, const void* v,
                         const void* d_o, const float* lse, const float* delta, float* dq,
                         void* stream);

/* A whole rank's ring, run natively: the schedule below with one cp_attn_step per visited
 * chunk (accumulating, or step + cp_attn_merge when o_work/lse_work are given). */
typedef struct {
  int32_t heads_q, heads_kv;
  int32_t chunk_len;   /* Lc: rows per chunk (the query shard is one chunk) */
  int32_t head_dim;
  int32_t n_cp;        /* ring size N_cp >= 1 */
  int32_t rank;        /* 0 <= rank < n_cp */
  int32_t causal;
  float scale;
  int32_t dtype;
} cp_ring_desc;

/*
 * cp_ring_schedule — the chunk held at each of the n_cp ring steps and its class. A rank
 * receives from rank - 1, so at step s it holds chunk (rank - s) mod n_cp. Classes:
 * 0 = every key visible, 1 = the rank's own chunk (triangular mask), 2 = skipped (causal and
 * the chunk is after the rank's own). chunks, classes: host arrays of n_cp int32.
 * Returns the number of visited (non-skipped) steps, or a negative cp_status.
 */
int32_t cp_ring_schedule(int32_t n_cp, int32_t rank, int32_t causal, int32_t* chunks,
                         int32_t* classes);

/*
 * cp_attn_ring_fwd — the rank's forward over all ring steps.
 *   q [heads_q, Lc, d]; k_chunks, v_chunks [n_cp, heads_kv, Lc, d] (chunk c at offset
 *   c * heads_kv * Lc * d elements); o [heads_q, Lc, d] fp32 and lse [heads_q, Lc] fp32 receive
 *   the final shard. o_work/lse_work: NULL for the fused fold, or scratch of o's/lse's size to
 *   run each step into scratch followed by cp_attn_merge.
 */
cp_status cp_attn_ring_fwd(const cp_ring_desc* ring, const void* q, const void* k_chunks,
                           const void* v_chunks, float* o, float* lse, float* o_work,
                           float* lse_work, void* stream);

/*
 * cp_attn_ring_bwd — the rank's backward over all ring steps: cp_attn_bwd_prep on (o, d_o),
 * then cp_attn_bwd for every visited chunk. o, lse: the final forward output of
 * cp_attn_ring_fwd. delta_work: [heads_q, Lc] fp32 scratch. dq [heads_q, Lc, d] and
 * dk_chunks, dv_chunks [n_cp, heads_kv, Lc, d] fp32 are accumulated (+=).
 */
cp_status cp_attn_ring_bwd(const cp_ring_desc* ring, const void* q, const void* k_chunks,
                           const void* v_chunks, const void* d_o, const float* o,
                           const float* lse, float* delta_work, float* dq, float* dk_chunks,
                           float* dv_chunks, void* stream);

/*
 * cp_attn_ring_bwd_noalloc — cp_attn_ring_bwd for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid allocation): the same
 * backward ring, with the per-row delta kept in a fixed device array of the library instead of
 * a caller-provided delta_work. Same arguments and results as cp_attn_ring_bwd otherwise.
 *  - Limit: heads_q * chunk_len <= CP_NOALLOC_MAX_ROWS rows (16 MiB of fp32 per device, held
 *    until the process ends); larger requests return CP_ERR_SCRATCH_LIMIT before anything is
 *    enqueued.
 *  - The array is per device and shared by every call on that device, so calls that overlap
 *    in time on one device (different streams or threads) race; serialize them. The array
 *    needs no clearing: each call overwrites the rows it reads.
 *  - Allocates nothing (no hipMalloc); the first call on a device looks the array up once.
 */
#define CP_NOALLOC_MAX_ROWS (1 << 22)
cp_status cp_attn_ring_bwd_noalloc(const cp_ring_desc* ring, const void* q, const void* k_chunks,
                                   const void* v_chunks, const void* d_o, const float* o,
                                   const float* lse, float* dq, float* dk_chunks,
                                   float* dv_chunks, void* stream);

/*
 * Zig-zag causal load balancing (context-parallelism page, section 5: Llama 3's split, which
 * StripedHyena 2 also trains with): the sequence is cut into 2 * n_cp half-chunks x_0 ..
 * x_{2 n_cp - 1} of Lh rows and rank r holds x_r and x_{2 n_cp - 1 - r}, so every rank gets the
 * same causal work. Layout of a rank's tensors is half-major: q, d_o, o, dq [2, heads, Lh, d]
 * (index 0 = x_r, 1 = x_{2 n_cp - 1 - r}); lse, delta [2, heads, Lh]; the chunk a rank passes
 * around is its pair of halves, so k_chunks, v_chunks, dk_chunks, dv_chunks are
 * [n_cp, 2, heads_kv, Lh, d]. ring->chunk_len is Lh (the half-chunk length).
 */

/* cp_zigzag_shards — the two half-chunk indices rank `rank` holds (shards[0] < shards[1]).
 * Returns 0, or a negative cp_status. Host only. */
int32_t cp_zigzag_shards(int32_t n_cp, int32_t rank, int32_t* shards);

/* cp_attn_ring_fwd_zigzag — the rank's forward over all ring steps under the zig-zag split:
 * at step s it holds rank (rank - s) mod n_cp's pair of halves and runs cp_attn_step for each
 * (query half, key/value half) pair that is not causally empty, folding into o/lse. */
cp_status cp_attn_ring_fwd_zigzag(const cp_ring_desc* ring, const void* q, const void* k_chunks,
                                  const void* v_chunks, float* o, float* lse, void* stream);

/* cp_attn_ring_bwd_zigzag — the matching backward: delta prep over both halves, then
 * cp_attn_bwd for every non-empty (query half, key/value half) pair. dq, dk_chunks, dv_chunks
 * are accumulated (+=). delta_work: [2, heads_q, Lh] fp32 scratch. */
cp_status cp_attn_ring_bwd_zigzag(const cp_ring_desc* ring, const void* q, const void* k_chunks,
                                  const void* v_chunks, const void* d_o, const float* o,
                                  const float* lse, float* delta_work, float* dq,
                                  float* dk_chunks, float* dv_chunks, void* stream);

/*
 * Striped ordering (context-parallelism page, section 5, after Brandon et al.): token t of the
 * sequence lives on rank t mod n_cp, so rank r holds tokens r, r + n_cp, r + 2 n_cp, ... and
 * every ring step is a (shifted) triangle of equal work. (The page's wording, "2 n_cp shards,
 * two per rank in stripes", is taken as garbled: that reading would not balance causal work.)
 * Within stripe coordinates query i of rank r sees key j of stripe c iff j <= i when c <= r and
 * j <= i - 1 when c > r, which is the step's causal test with q_pos0 = 0 and kv_pos0 = (c > r).
 * Layout as for the contiguous ring: q [heads_q, Ls, d] (the rank's stripe, Ls = L / n_cp),
 * k_chunks/v_chunks [n_cp, heads_kv, Ls, d] (stripe c at index c), o [heads_q, Ls, d], lse
 * [heads_q, Ls]; ring->chunk_len is Ls.
 */
cp_status cp_attn_ring_fwd_striped(const cp_ring_desc* ring, const void* q,
                                   const void* k_chunks, const void* v_chunks, float* o,
                                   float* lse, void* stream);
cp_status cp_attn_ring_bwd_striped(const cp_ring_desc* ring, const void* q,
                                   const void* k_chunks, const void* v_chunks, const void* d_o,
                                   const float* o, const float* lse, float* delta_work,
                                   float* dq, float* dk_chunks, float* dv_chunks, void* stream);

/* Static description of a status code (never NULL). */
const char* cp_attn_status_string(int32_t status);

/* ABI version of this header: increments on any incompatible change. */
int32_t cp_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CP_ATTN_H */
