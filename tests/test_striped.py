"""Striped ordering (token t on rank t mod N_cp; after Brandon et al., as cited on the
context-parallelism page, section 5).

CPU: the stripe-local causal test the ring driver relies on (query i of rank r sees key j of
stripe c iff j - i <= q_pos0 - kv_pos0 with q_pos0 = 0, kv_pos0 = [c > r]) equals the global
test on positions r + N i and c + N j, by brute force; and each rank's visible-pair count has
the closed form sum_i (r + N i + 1), so ranks differ by under N keys a query row.
GPU: the striped ring forward and backward against the oracle's full-sequence attention.
"""
import numpy as np
import pytest

import oracle
from long_context_sequence_amd import inputs


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8])
def test_stripe_local_mask_equals_global_causality(n):
    ls = 7
    for r in range(n):
        work = 0
        for c in range(n):
            local = oracle.visibility(ls, ls, q_pos0=0, kv_pos0=int(c > r), causal=True)
            qpos = r + n * np.arange(ls)
            kpos = c + n * np.arange(ls)
            glob = kpos[None, :] <= qpos[:, None]
            assert np.array_equal(local, glob), (n, r, c)
            work += int(glob.sum())
        # query r + N i sees r + N i + 1 keys: ranks differ by at most N - 1 keys a row
        assert work == sum(r + n * i + 1 for i in range(ls))


@pytest.mark.gpu
def test_striped_ring_matches_oracle():
    import torch

    from long_context_sequence_amd import binding as cp
    from util import GRAD_REL, check_o_lse

    n, hq, hkv, ls, d = 4, 4, 2, 96, 128
    L = n * ls
    key = 501
    qf = inputs.make(key, "q", 0, (hq, L, d), "bf16")     # natural order, all ranks
    kf = inputs.make(key, "k", 0, (hkv, L, d), "bf16")
    vf = inputs.make(key, "v", 0, (hkv, L, d), "bf16")
    dof = inputs.make(key, "do", 0, (hq, L, d), "bf16")
    stripe = lambda a, r: np.ascontiguousarray(a[:, r::n])  # noqa: E731
    kd = inputs.to_torch(np.stack([stripe(kf, c) for c in range(n)]), "cuda")
    vd = inputs.to_torch(np.stack([stripe(vf, c) for c in range(n)]), "cuda")
    Q, K, V, DO = (inputs.widen(a) for a in (qf, kf, vf, dof))
    o_full, l_full = oracle.attention_forward(Q, K, V, causal=True)
    for r in range(n):
        q = inputs.to_torch(stripe(qf, r), "cuda")
        d_o = inputs.to_torch(stripe(dof, r), "cuda")
        o = torch.empty(q.shape, device="cuda")
        lse = torch.empty(q.shape[:2], device="cuda")
        cp.ring_fwd_striped(q, kd, vd, o, lse, r, True)
        delta = torch.empty_like(lse)
        dq = torch.zeros_like(o)
        dk = torch.zeros(kd.shape, device="cuda")
        dv = torch.zeros(vd.shape, device="cuda")
        cp.ring_bwd_striped(q, kd, vd, d_o, o, lse, delta, dq, dk, dv, r, True)
        torch.cuda.synchronize()
        check_o_lse(o.cpu().numpy(), lse.cpu().numpy(), o_full[:, r::n], l_full[:, r::n], "bf16",
                    f"striped rank {r}")
        # this rank's gradient contribution: dO zero on every other rank's rows
        do_r = np.zeros_like(DO)
        do_r[:, r::n] = DO[:, r::n]
        gq, gk, gv = oracle.attention_backward(Q, K, V, do_r, causal=True)
        for name, got, ref in (("dQ", dq.cpu().numpy(), gq[:, r::n]),
                               ("dK", dk.cpu().numpy(), np.stack([gk[:, c::n] for c in range(n)])),
                               ("dV", dv.cpu().numpy(), np.stack([gv[:, c::n] for c in range(n)]))):
            assert np.max(np.abs(got - ref)) <= GRAD_REL * np.max(np.abs(ref)), f"{name} rank {r}"
