"""Plain fp64 CPU oracle for one context-parallel rank's ring attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import this module. The GPU library never calls it and shares no code with it.

What the ring computes (StripedHyena 2 context-parallelism page, section 2, "ring attention:
passing key/value around the ring"): a rank keeps its query shard, receives every key/value
chunk once, folds each partial result in with online softmax statistics, and after N_cp steps
holds its shard of *full* attention, obtained without gathering the sequence in one place.
The oracle therefore is the plain definition of full softmax attention over the concatenated
sequence. It contains no chunking and no online softmax: a row's scores are formed at once,
its log-sum-exp is taken, and the normalised weights multiply V.

Readings of points the pages leave open (each also listed in the design notes):
  * scale: scores are q.k / sqrt(d) unless a scale is given;
  * LSE: natural logarithm of the sum of exp(scaled score) over the visible keys;
  * causal masking (causal-model load-balancing section of the same page, which only says the
    work is triangular): a query at global position p sees keys at global positions <= p,
    itself included; positions are chunk_index * chunk_len + local index (contiguous chunks);
  * GQA (2D-attention summary, LLM-architecture section; Ulysses explainer, ring-vs-Ulysses
    section): query head h reads key/value head h // (H_q / H_kv) (contiguous groups);
  * a row with no visible key has O = 0 and LSE = -inf.

Backward (the pages give none): loss = sum(O * dO); the softmax Jacobian
diag(p) - p p^T is applied to dP = dO V^T row by row, the textbook derivation, not the
D = rowsum(dO * O) shortcut used by fast kernels.

Every function is pinned by tests that do not re-type these formulas: closed forms, invariants,
torch's CPU scaled_dot_product_attention with an explicit mask and its autograd, and central
finite differences.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q, k, v):
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("q, k, v must be [heads, len, d]")
    hq, _, d = q.shape
    hkv, lk, dk = k.shape
    if v.shape[:2] != k.shape[:2] or dk != d:
        raise ValueError("k must be [H_kv, L_kv, d] with the query's d, v [H_kv, L_kv, d_v]")
    if hkv == 0 or hq % hkv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    return hq, hkv, hq // hkv, d


def _default_scale(scale, d):
    return 1.0 / np.sqrt(d) if scale is None or scale <= 0 else float(scale)


def visibility(lq, lk, q_pos0=0, kv_pos0=0, causal=False):
    """Boolean [lq, lk]: may the query at q_pos0+i attend to the key at kv_pos0+j."""
    if not causal:
        return np.ones((lq, lk), dtype=bool)
    qp = q_pos0 + np.arange(lq, dtype=np.int64)
    kp = kv_pos0 + np.arange(lk, dtype=np.int64)
    return kp[None, :] <= qp[:, None]


def _row_block_softmax(s):
    """Row-wise log-sum-exp and normalised weights of scores s (masked entries are -inf)."""
    m = np.max(s, axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    tot = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, tot)))
    p = np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, tot)[:, None])
    return lse, p


def attention_forward(q, k, v, q_pos0=0, kv_pos0=0, causal=False, scale=None, row_block=512):
    """Full softmax attention of q [H_q, L_q, d] over k, v [H_kv, L_kv, d], in fp64.

    Returns O [H_q, L_q, d] and LSE [H_q, L_q]. Row blocks only bound memory: each row's
    softmax is over all of its visible keys at once.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    hq, hkv, grp, d = _check_shapes(q, k, v)
    lq, lk = q.shape[1], k.shape[1]
    sc = _default_scale(scale, d)
    o = np.zeros((hq, lq, v.shape[2]))
    lse = np.full((hq, lq), -np.inf)
    for h in range(hq):
        g = h // grp
        for i0 in range(0, lq, row_block):
            i1 = min(lq, i0 + row_block)
            s = sc * (q[h, i0:i1] @ k[g].T)
            vis = visibility(i1 - i0, lk, q_pos0 + i0, kv_pos0, causal)
            s = np.where(vis, s, -np.inf)
            lse[h, i0:i1], p = _row_block_softmax(s)
            o[h, i0:i1] = p @ v[g]
    return o, lse


def attention_rows(q_rows, k, v, q_heads, rows, heads_q, q_pos0=0, kv_pos0=0, causal=False,
                   scale=None):
    """O and LSE for selected query rows only, one row at a time (same definition as
    attention_forward). q_rows[t] is row rows[t] of query head q_heads[t] of a shard with
    heads_q heads whose row 0 sits at global position q_pos0; k, v are the full key/value
    tensors [H_kv, L_kv, d] starting at kv_pos0. Returns O [n, d] and LSE [n]."""
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    q_heads = np.asarray(q_heads, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    hkv, lk, d = k.shape
    if heads_q % hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    grp = heads_q // hkv
    sc = _default_scale(scale, d)
    n = q_rows.shape[0]
    o = np.zeros((n, d))
    lse = np.full(n, -np.inf)
    kp = kv_pos0 + np.arange(lk, dtype=np.int64)
    for t in range(n):
        g = int(q_heads[t]) // grp
        s = sc * (k[g] @ q_rows[t])
        if causal:
            s = np.where(kp <= q_pos0 + rows[t], s, -np.inf)
        l1, p = _row_block_softmax(s[None, :])
        lse[t] = l1[0]
        o[t] = p[0] @ v[g]
    return o, lse


def merge(o_a, lse_a, o_b, lse_b):
    """Fold two partial results over disjoint key sets into the result over their union.

    With a = LSE_a and b = LSE_b (natural log): LSE = max(a, b) + log(1 + exp(-|a - b|)),
    O = exp(a - LSE) O_a + exp(b - LSE) O_b. Both empty (a = b = -inf) gives (0, -inf).
    This is the online-softmax accumulation of the ring-attention steps, written for two
    operands (context-parallelism page, section 2, ring attention step 3).
    """
    o_a, lse_a, o_b, lse_b = _f64(o_a), _f64(lse_a), _f64(o_b), _f64(lse_b)
    hi = np.maximum(lse_a, lse_b)
    both_empty = np.isneginf(hi)
    hi_safe = np.where(both_empty, 0.0, hi)
    with np.errstate(invalid="ignore"):
        gap = np.where(both_empty, 0.0, np.abs(lse_a - lse_b))
    gap = np.where(np.isnan(gap), np.inf, gap)
    lse = np.where(both_empty, -np.inf, hi_safe + np.log1p(np.exp(-gap)))
    lse_safe = np.where(both_empty, 0.0, lse)
    wa = np.where(both_empty, 0.0, np.exp(lse_a - lse_safe))
    wb = np.where(both_empty, 0.0, np.exp(lse_b - lse_safe))
    return wa[..., None] * o_a + wb[..., None] * o_b, lse


def attention_backward(q, k, v, d_o, q_pos0=0, kv_pos0=0, causal=False, scale=None,
                       row_block=512):
    """Gradients of loss = sum(O * dO) for the attention of attention_forward, in fp64.

    For each query head h (key/value head g = h // group) and visible pair (i, j):
      P_ij  = exp(s_ij - LSE_i)
      dP_ij = dO_i . V_j
      dS_ij = P_ij * (dP_ij - sum_k P_ik dP_ik)          (softmax Jacobian)
      dQ_i += scale * sum_j dS_ij K_j
      dK_j += scale * sum_i dS_ij Q_i                      (summed over the group's heads)
      dV_j += sum_i P_ij dO_i                              (summed over the group's heads)
    Returns dQ [H_q, L_q, d], dK and dV [H_kv, L_kv, d].
    """
    q, k, v, d_o = _f64(q), _f64(k), _f64(v), _f64(d_o)
    hq, hkv, grp, d = _check_shapes(q, k, v)
    if d_o.shape != q.shape:
        raise ValueError("dO must match q")
    lq, lk = q.shape[1], k.shape[1]
    sc = _default_scale(scale, d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(hq):
        g = h // grp
        for i0 in range(0, lq, row_block):
            i1 = min(lq, i0 + row_block)
            s = sc * (q[h, i0:i1] @ k[g].T)
            vis = visibility(i1 - i0, lk, q_pos0 + i0, kv_pos0, causal)
            s = np.where(vis, s, -np.inf)
            _, p = _row_block_softmax(s)
            dp = d_o[h, i0:i1] @ v[g].T
            jac = (p * dp).sum(axis=1, keepdims=True)
            ds = p * (dp - jac)
            dq[h, i0:i1] += sc * (ds @ k[g])
            dk[g] += sc * (ds.T @ q[h, i0:i1])
            dv[g] += p.T @ d_o[h, i0:i1]
    return dq, dk, dv


def attention_backward_rows(q_rows, do_rows, k, v, q_heads, rows, heads_q, q_pos0=0,
                            kv_pos0=0, causal=False, scale=None, keys=None):
    """attention_backward restricted to selected query rows, for checks at sizes where the full
    gradient is out of reach: q_rows[t], do_rows[t] are row rows[t] of query head q_heads[t] (a
    shard of heads_q heads whose row 0 is at global position q_pos0); k, v [H_kv, L_kv, d] are
    the full key/value tensors starting at kv_pos0. Each row's softmax, dP and Jacobian term
    run over all of its visible keys, as in attention_backward.

    Returns dQ of the rows [n, d] and, when `keys` (indices along L_kv) is given, the selected
    rows' contributions to dK and dV at those keys, [H_kv, len(keys), d] each: the complete
    dK/dV there when the rows include every row that sees those keys."""
    q_rows, do_rows = _f64(q_rows), _f64(do_rows)
    q_heads = np.asarray(q_heads, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    hkv, lk, d = k.shape
    if heads_q % hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    grp = heads_q // hkv
    sc = _default_scale(scale, d)
    keys = None if keys is None else np.asarray(keys, dtype=np.int64)
    dq = np.zeros_like(q_rows)
    nk = 0 if keys is None else len(keys)
    dk = np.zeros((hkv, nk, d))
    dv = np.zeros((hkv, nk, v.shape[2]))
    for g in np.unique(q_heads // grp):
        sel = np.nonzero(q_heads // grp == g)[0]
        kg, vg = _f64(k[g]), _f64(v[g])
        s = sc * (q_rows[sel] @ kg.T)
        if causal:
            vis = (kv_pos0 + np.arange(lk))[None, :] <= (q_pos0 + rows[sel])[:, None]
            s = np.where(vis, s, -np.inf)
        _, p = _row_block_softmax(s)
        dp = do_rows[sel] @ vg.T
        jac = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - jac)
        dq[sel] = sc * (ds @ kg)
        if nk:
            dk[g] += sc * (ds[:, keys].T @ q_rows[sel])
            dv[g] += p[:, keys].T @ do_rows[sel]
    return dq, dk, dv


def softmax_dot(q, k, v, d_o, q_pos0=0, kv_pos0=0, causal=False, scale=None, row_block=512):
    """sum_j P_ij dP_ij per (head, row) [H_q, L_q]: the Jacobian term of attention_backward.

    A kernel's D = rowsum(dO * O) must equal this (since O_i = sum_j P_ij V_j)."""
    q, k, v, d_o = _f64(q), _f64(k), _f64(v), _f64(d_o)
    hq, hkv, grp, d = _check_shapes(q, k, v)
    lq, lk = q.shape[1], k.shape[1]
    sc = _default_scale(scale, d)
    out = np.zeros((hq, lq))
    for h in range(hq):
        g = h // grp
        for i0 in range(0, lq, row_block):
            i1 = min(lq, i0 + row_block)
            s = sc * (q[h, i0:i1] @ k[g].T)
            vis = visibility(i1 - i0, lk, q_pos0 + i0, kv_pos0, causal)
            _, p = _row_block_softmax(np.where(vis, s, -np.inf))
            out[h, i0:i1] = (p * (d_o[h, i0:i1] @ v[g].T)).sum(axis=1)
    return out


def rank_forward(q_rank, k_chunks, v_chunks, rank, causal, scale=None):
    """The rank's final shard: full attention of its queries over the concatenated chunks.

    q_rank [H_q, L_c, d]; k_chunks, v_chunks [N_cp, H_kv, L_c, d]. Query positions start at
    rank * L_c; the concatenated keys start at 0.
    """
    k_full = np.concatenate(list(_f64(k_chunks)), axis=1)
    v_full = np.concatenate(list(_f64(v_chunks)), axis=1)
    lc = q_rank.shape[1]
    return attention_forward(q_rank, k_full, v_full, q_pos0=rank * lc, kv_pos0=0,
                             causal=causal, scale=scale)


def rank_backward(q_rank, k_chunks, v_chunks, d_o, rank, causal, scale=None):
    """This rank's gradient contribution: dQ of its shard and dK/dV split back per chunk."""
    n = len(k_chunks)
    k_full = np.concatenate(list(_f64(k_chunks)), axis=1)
    v_full = np.concatenate(list(_f64(v_chunks)), axis=1)
    lc = q_rank.shape[1]
    dq, dk, dv = attention_backward(q_rank, k_full, v_full, d_o, q_pos0=rank * lc, kv_pos0=0,
                                    causal=causal, scale=scale)
    split = lambda t: np.stack(np.split(t, n, axis=1))  # noqa: E731
    return dq, split(dk), split(dv)
