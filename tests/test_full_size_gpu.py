"""The named workloads at full size against the fp64 oracle, in the launch configuration the
benchmark times, through the C ABI.

What is checked is the ring's end state (StripedHyena 2 context-parallelism page, section 2,
ring attention step 4): after its N_cp steps a rank holds its shard of full attention. So every
output is compared with full softmax attention over the concatenated sequence:

* 8K MHA causal: all 8 ranks, every head and row, O and LSE element by element;
* 32K GQA causal with RMS-normalised rows: rank 7 in full;
* 32K GQA causal forward + backward: rank 7's O and LSE, dQ, and dK/dV of all 8 chunks, for
  every key/value head group;
* 208K shard (rank 15 of 16): 1,024 seeded rows (rows 0, 1 and the last row included) for O,
  LSE and dQ, each over its up to 212,992 visible keys; softmax rows summing to one with the
  GPU's LSE on every sampled row; dK/dV of the diagonal chunk's last keys; gradient-sum
  identities over every key.

The oracle runs per head (or per block of rows) on the host cores in a thread pool.
"""
import numpy as np
import pytest
import torch

import oracle
from long_context_sequence_amd import binding as cp
from long_context_sequence_amd import configs, inputs

from util import GRAD_REL, check_o_lse, oracle_map, sample_rows

pytestmark = pytest.mark.gpu


def _check_grad(got, ref, name):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = float(np.max(np.abs(got - ref)))
    scale = float(np.max(np.abs(ref)))
    assert err <= GRAD_REL * scale, f"{name}: max|d| {err:.3g} vs max|ref| {scale:.3g}"
    return err / scale


def _keys_host(wl):
    """Every chunk of K and V concatenated along the sequence: [H_kv, L, d] fp32 (exact)."""
    k_host = inputs.workload_kv(wl, "k")
    v_host = inputs.workload_kv(wl, "v")
    kf = np.concatenate([inputs.bf16_bits_to_f32(c) for c in k_host], axis=1)
    vf = np.concatenate([inputs.bf16_bits_to_f32(c) for c in v_host], axis=1)
    return k_host, v_host, kf, vf


def _ring_forward(q, kd, vd, rank, causal):
    o = torch.empty(q.shape, device="cuda")
    lse = torch.empty(q.shape[:2], device="cuda")
    cp.ring_fwd(q, kd, vd, o, lse, rank, causal)
    return o, lse


def _oracle_forward_per_head(wl, qf, kf, vf, rank):
    """Full attention of the rank's shard over the whole sequence, one task per query head."""
    lc = wl.chunk_len

    def head(h):
        g = h // wl.group
        return oracle.attention_forward(qf[h:h + 1], kf[g:g + 1], vf[g:g + 1], q_pos0=rank * lc,
                                        causal=wl.causal, scale=wl.scale)

    res = oracle_map(head, range(wl.heads_q))
    return np.concatenate([o for o, _ in res]), np.concatenate([lse for _, lse in res])


@pytest.mark.timeout(900)
def test_mha_8k_every_rank_in_full():
    wl = configs.C2
    k_host, v_host, kf, vf = _keys_host(wl)
    kd, vd = inputs.to_torch(k_host, "cuda"), inputs.to_torch(v_host, "cuda")
    for r in wl.ranks:
        qa = inputs.workload_tensor(wl, "q", r)
        o, lse = _ring_forward(inputs.to_torch(qa, "cuda"), kd, vd, r, wl.causal)
        torch.cuda.synchronize()
        o_ref, lse_ref = _oracle_forward_per_head(wl, inputs.bf16_bits_to_f32(qa), kf, vf, r)
        e_o, e_l = check_o_lse(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16",
                               f"8K MHA rank {r}")
        print(f"8K MHA rank {r}: max|dO| {e_o:.2e} max|dLSE| {e_l:.2e}", flush=True)


@pytest.mark.timeout(900)
def test_gqa_32k_rms_last_rank_in_full():
    wl = configs.C3
    r = wl.ranks[-1]
    k_host, v_host, kf, vf = _keys_host(wl)
    kd, vd = inputs.to_torch(k_host, "cuda"), inputs.to_torch(v_host, "cuda")
    qa = inputs.workload_tensor(wl, "q", r)
    o, lse = _ring_forward(inputs.to_torch(qa, "cuda"), kd, vd, r, wl.causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle_forward_per_head(wl, inputs.bf16_bits_to_f32(qa), kf, vf, r)
    e_o, e_l = check_o_lse(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16",
                           f"32K GQA RMS rank {r}")
    print(f"32K GQA RMS rank {r}: max|dO| {e_o:.2e} max|dLSE| {e_l:.2e}", flush=True)


@pytest.mark.timeout(900)
def test_gqa_32k_forward_backward_every_head_group_in_full():
    wl = configs.C5
    r = wl.ranks[-1]
    lc, grp, n = wl.chunk_len, wl.group, wl.n_cp
    k_host, v_host, kf, vf = _keys_host(wl)
    qa = inputs.workload_tensor(wl, "q", r)
    da = inputs.workload_tensor(wl, "do", r)
    q, d_o = inputs.to_torch(qa, "cuda"), inputs.to_torch(da, "cuda")
    kd, vd = inputs.to_torch(k_host, "cuda"), inputs.to_torch(v_host, "cuda")
    o, lse = _ring_forward(q, kd, vd, r, True)
    delta = torch.empty_like(lse)
    dq = torch.zeros_like(o)
    dk = torch.zeros(kd.shape, device="cuda")
    dv = torch.zeros(vd.shape, device="cuda")
    cp.ring_bwd(q, kd, vd, d_o, o, lse, delta, dq, dk, dv, r, True)
    torch.cuda.synchronize()
    o, lse, dq = o.cpu().numpy(), lse.cpu().numpy(), dq.cpu().numpy()
    # [N_cp, H_kv, Lc, d] -> [H_kv, L, d]: the chunks in sequence order
    dk = dk.permute(1, 0, 2, 3).reshape(wl.heads_kv, n * lc, -1).cpu().numpy()
    dv = dv.permute(1, 0, 2, 3).reshape(wl.heads_kv, n * lc, -1).cpu().numpy()
    qf, dof = inputs.bf16_bits_to_f32(qa), inputs.bf16_bits_to_f32(da)

    def head(h):
        g = h // grp
        args = (qf[h:h + 1], kf[g:g + 1], vf[g:g + 1])
        o_h, l_h = oracle.attention_forward(*args, q_pos0=r * lc, causal=True, scale=wl.scale)
        dq_h, dk_h, dv_h = oracle.attention_backward(*args, dof[h:h + 1], q_pos0=r * lc,
                                                     causal=True, scale=wl.scale)
        return o_h, l_h, dq_h, dk_h, dv_h

    res = oracle_map(head, range(wl.heads_q))
    o_ref = np.concatenate([x[0] for x in res])
    lse_ref = np.concatenate([x[1] for x in res])
    dq_ref = np.concatenate([x[2] for x in res])
    e_o, e_l = check_o_lse(o, lse, o_ref, lse_ref, "bf16", "32K fwd+bwd forward")
    e_q = _check_grad(dq, dq_ref, "dQ")
    worst = [e_q, 0.0, 0.0]
    for g in range(wl.heads_kv):
        dk_ref = sum(res[h][3][0] for h in range(g * grp, (g + 1) * grp))
        dv_ref = sum(res[h][4][0] for h in range(g * grp, (g + 1) * grp))
        worst[0] = max(worst[0], _check_grad(dq[g * grp:(g + 1) * grp],
                                             dq_ref[g * grp:(g + 1) * grp], f"dQ group {g}"))
        worst[1] = max(worst[1], _check_grad(dk[g], dk_ref, f"dK group {g}"))
        worst[2] = max(worst[2], _check_grad(dv[g], dv_ref, f"dV group {g}"))
    print(f"32K fwd+bwd rank {r}: max|dO| {e_o:.2e} max|dLSE| {e_l:.2e}; scaled gradient "
          f"errors dQ {worst[0]:.2e} dK {worst[1]:.2e} dV {worst[2]:.2e}", flush=True)


def _row_blocks(heads, rows, group, size=32):
    """Indices of the sampled rows, grouped by key/value head, in blocks of at most `size`."""
    out = []
    kv = heads // group
    for g in np.unique(kv):
        idx = np.nonzero(kv == g)[0]
        out += [idx[i:i + size] for i in range(0, idx.size, size)]
    return out


@pytest.mark.timeout(900)
def test_208k_shard_1024_rows_forward_backward():
    wl = configs.C4
    r = wl.ranks[-1]
    lc, grp = wl.chunk_len, wl.group
    qa = inputs.workload_tensor(wl, "q", r)
    da = inputs.workload_tensor(wl, "do", r)
    k_host = inputs.workload_kv(wl, "k")
    v_host = inputs.workload_kv(wl, "v")
    q, d_o = inputs.to_torch(qa, "cuda"), inputs.to_torch(da, "cuda")
    k, v = inputs.to_torch(k_host, "cuda"), inputs.to_torch(v_host, "cuda")
    o, lse = _ring_forward(q, k, v, r, True)
    delta = torch.empty_like(lse)
    dq = torch.zeros_like(o)
    dk = torch.zeros(k.shape, device="cuda")
    dv = torch.zeros(v.shape, device="cuda")
    cp.ring_bwd(q, k, v, d_o, o, lse, delta, dq, dk, dv, r, True)
    torch.cuda.synchronize()
    del k, v
    kf = np.concatenate([inputs.widen(c) for c in k_host], axis=1)   # [H_kv, L, d] fp64
    vf = np.concatenate([inputs.widen(c) for c in v_host], axis=1)
    del k_host, v_host
    qf, dof = inputs.widen(qa), inputs.widen(da)

    heads, rows = sample_rows(wl, r, 1024, seed=415)
    assert {0, 1, lc - 1} <= set(rows.tolist())
    o_s = o[heads, rows].cpu().numpy()
    l_s = lse[heads, rows].cpu().numpy()
    dq_s = dq[heads, rows].cpu().numpy()

    def block(idx):
        hb, rb = heads[idx], rows[idx]
        o_ref, l_ref = oracle.attention_rows(qf[hb, rb], kf, vf, hb, rb, wl.heads_q,
                                             q_pos0=r * lc, causal=True, scale=wl.scale)
        dq_ref, _, _ = oracle.attention_backward_rows(qf[hb, rb], dof[hb, rb], kf, vf, hb, rb,
                                                      wl.heads_q, q_pos0=r * lc, causal=True,
                                                      scale=wl.scale)
        # softmax rows sum to one with the GPU's LSE: sum_j exp(s_ij - LSE_i) over visible keys
        sums = np.empty(idx.size)
        for t, (h, i) in enumerate(zip(hb, rb)):
            nvis = r * lc + i + 1
            s = (kf[h // grp, :nvis] @ qf[h, i]) * wl.scale
            sums[t] = np.sum(np.exp(s - l_s[idx[t]]))
        return idx, o_ref, l_ref, dq_ref, sums

    o_ref = np.empty_like(o_s, dtype=np.float64)
    l_ref = np.empty_like(l_s, dtype=np.float64)
    dq_ref = np.empty_like(dq_s, dtype=np.float64)
    sums = np.empty(heads.size)
    for idx, ob, lb, qb, sb in oracle_map(block, _row_blocks(heads, rows, grp)):
        o_ref[idx], l_ref[idx], dq_ref[idx], sums[idx] = ob, lb, qb, sb
    e_o, e_l = check_o_lse(o_s, l_s, o_ref, l_ref, "bf16", "208K shard, 1,024 rows")
    e_q = _check_grad(dq_s, dq_ref, "dQ (1,024 rows)")
    e_sum = float(np.max(np.abs(sums - 1.0)))
    assert e_sum < 2e-3, f"rows sum to 1 with the GPU's LSE: worst {e_sum:.3g}"

    # dK/dV of the diagonal chunk's last 24 keys of one key/value head: only the shard's last 24
    # rows of that head's 4 query heads see them, so the row-restricted oracle is complete there
    g, n_tail = 5, 24
    keys = r * lc + np.arange(lc - n_tail, lc)
    hh, rr = np.meshgrid(np.arange(g * grp, (g + 1) * grp), np.arange(lc - n_tail, lc),
                         indexing="ij")
    hh, rr = hh.ravel(), rr.ravel()
    _, dk_ref, dv_ref = oracle.attention_backward_rows(qf[hh, rr], dof[hh, rr], kf, vf, hh, rr,
                                                       wl.heads_q, q_pos0=r * lc, causal=True,
                                                       scale=wl.scale, keys=keys)
    e_k = _check_grad(dk[r, g, lc - n_tail:].cpu().numpy(), dk_ref[g], "dK (diagonal tail keys)")
    e_v = _check_grad(dv[r, g, lc - n_tail:].cpu().numpy(), dv_ref[g], "dV (diagonal tail keys)")
    print(f"208K shard: max|dO| {e_o:.2e} max|dLSE| {e_l:.2e} rows-sum {e_sum:.2e}; scaled "
          f"gradient errors dQ {e_q:.2e} dK {e_k:.2e} dV {e_v:.2e}", flush=True)

    # identities over every key of every chunk, per key/value head:
    # sum_j dV_j = sum over the group's rows of dO, and sum_j dK_j = 0 (rows of dS sum to 0)
    dk_sum = dk.double().sum(dim=(0, 2)).cpu().numpy()          # [H_kv, d]
    dv_sum = dv.double().sum(dim=(0, 2)).cpu().numpy()
    do_sum = dof.reshape(wl.heads_kv, grp * lc, -1).sum(axis=1)
    assert np.max(np.abs(dv_sum - do_sum)) <= 1e-3 * np.max(np.abs(do_sum))
    dk_max = float(dk.abs().max())
    assert np.max(np.abs(dk_sum)) <= 2e-2 * dk_max * np.sqrt(wl.n_cp * lc)
