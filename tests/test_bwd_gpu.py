"""Backward parity on the GPU: cp_attn_bwd_prep + cp_attn_bwd (and the native ring driver)
against the fp64 oracle's textbook-Jacobian gradients on the same seeded inputs.

Bar: per gradient tensor, max|g - g_ref| <= 5e-2 * max|g_ref| (gradients include the 1/sqrt(d)
chain-rule factor; at long sequences the gradients are far below 5e-2 in absolute terms, so the
bar is scaled by the reference's magnitude). Absolute errors are reported in the failure text.
"""
import numpy as np
import pytest
import torch

import oracle
from long_context_sequence_amd import binding as cp
from long_context_sequence_amd import inputs

from util import GRAD_REL, device_inputs, host_inputs, small_workload

pytestmark = pytest.mark.gpu


def _check_grad(got, ref, name):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = float(np.max(np.abs(got - ref)))
    scale = float(np.max(np.abs(ref)))
    assert err <= GRAD_REL * scale, f"{name}: max|d| {err:.3g} vs max|ref| {scale:.3g}"
    return err / scale


def _ring_fwd_bwd(wl, rank):
    q, k, v, d_o = device_inputs(wl, rank, with_do=True)
    o = torch.empty(q.shape, device="cuda")
    lse = torch.empty(q.shape[:2], device="cuda")
    cp.ring_fwd(q, k, v, o, lse, rank, wl.causal)
    delta = torch.empty_like(lse)
    dq = torch.zeros_like(o)
    dk = torch.zeros(k.shape, device="cuda")
    dv = torch.zeros(v.shape, device="cuda")
    cp.ring_bwd(q, k, v, d_o, o, lse, delta, dq, dk, dv, rank, wl.causal)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_small_ragged_gqa_all_ranks(d, causal):
    # 200-row chunks: ragged against the 64-row query tiles, the 128-key dK/dV tiles and the
    # 64-key dQ tiles; GQA group 2.
    wl = small_workload(201, "bf16", 4, 2, d, 200, 3, causal, backward=True)
    for r in range(wl.n_cp):
        dq, dk, dv = _ring_fwd_bwd(wl, r)
        q, k, v, do = host_inputs(wl, r, with_do=True)
        dq_ref, dk_ref, dv_ref = oracle.rank_backward(q, k, v, do, r, causal)
        _check_grad(dq, dq_ref, f"dQ rank {r}")
        _check_grad(dk, dk_ref, f"dK rank {r}")
        _check_grad(dv, dv_ref, f"dV rank {r}")
        if causal:  # chunks after the rank's own receive nothing
            assert np.all(dk[r + 1:] == 0) and np.all(dv[r + 1:] == 0)


@pytest.mark.parametrize("causal", [True, False])
def test_single_chunk_ring(causal):
    """N_cp = 1: the backward ring is one step over the whole sequence."""
    wl = small_workload(206, "bf16", 4, 2, 128, 300, 1, causal, backward=True)
    dq, dk, dv = _ring_fwd_bwd(wl, 0)
    q, k, v, do = host_inputs(wl, 0, with_do=True)
    dq_ref, dk_ref, dv_ref = oracle.rank_backward(q, k, v, do, 0, causal)
    _check_grad(dq, dq_ref, "dQ")
    _check_grad(dk, dk_ref, "dK")
    _check_grad(dv, dv_ref, "dV")


@pytest.mark.parametrize("hq,hkv", [(8, 1), (3, 3)])
def test_head_groupings(hq, hkv):
    """Multi-query (8 query heads share one key/value head: dK/dV sum over all 8) and odd-count
    multi-head attention, 136-row chunks."""
    wl = small_workload(203, "bf16", hq, hkv, 128, 136, 3, True, backward=True)
    for r in range(wl.n_cp):
        dq, dk, dv = _ring_fwd_bwd(wl, r)
        q, k, v, do = host_inputs(wl, r, with_do=True)
        dq_ref, dk_ref, dv_ref = oracle.rank_backward(q, k, v, do, r, True)
        _check_grad(dq, dq_ref, f"dQ rank {r}")
        _check_grad(dk, dk_ref, f"dK rank {r}")
        _check_grad(dv, dv_ref, f"dV rank {r}")


@pytest.mark.parametrize("q0,k0,causal", [
    (0, 0, True),        # diagonal
    (400, 0, True),      # fully visible
    (0, 0, False),
    (40, 100, True),     # the first 60 rows see nothing (LSE = -inf)
])
def test_single_step_with_offsets(q0, k0, causal):
    hq, hkv, d, lq, lk = 6, 2, 128, 150, 170
    qa = inputs.make(202, "q", 0, (hq, lq, d), "bf16")
    ka = inputs.make(202, "k", 0, (hkv, lk, d), "bf16")
    va = inputs.make(202, "v", 0, (hkv, lk, d), "bf16")
    da = inputs.make(202, "do", 0, (hq, lq, d), "bf16")
    q, k, v, d_o = (inputs.to_torch(a, "cuda") for a in (qa, ka, va, da))
    o = torch.empty(q.shape, device="cuda")
    lse = torch.empty(q.shape[:2], device="cuda")
    assert cp.step(q, k, v, o, lse, q_pos0=q0, kv_pos0=k0, causal=causal) == cp.CP_OK
    delta = torch.empty_like(lse)
    cp.bwd_prep(o, d_o, delta)
    dq = torch.zeros_like(o)
    dk = torch.zeros(k.shape, device="cuda")
    dv = torch.zeros(v.shape, device="cuda")
    assert cp.bwd(q, k, v, d_o, lse, delta, dq, dk, dv, q_pos0=q0, kv_pos0=k0,
                  causal=causal) == cp.CP_OK
    torch.cuda.synchronize()
    ref = oracle.attention_backward(*(inputs.widen(a) for a in (qa, ka, va, da)), q_pos0=q0,
                                    kv_pos0=k0, causal=causal)
    for name, got, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        _check_grad(got.cpu().numpy(), r, name)
    if (q0, k0) == (40, 100):
        assert bool((dq[:, :60] == 0).all())


def test_accumulates_into_existing_gradients():
    wl = small_workload(203, "bf16", 4, 2, 128, 128, 2, True, backward=True)
    q, k, v, d_o = device_inputs(wl, 1, with_do=True)
    o = torch.empty(q.shape, device="cuda")
    lse = torch.empty(q.shape[:2], device="cuda")
    cp.ring_fwd(q, k, v, o, lse, 1, True)
    delta = torch.empty_like(lse)
    grads = []
    for init in (0.0, 1.5):
        dq = torch.full(q.shape, init, device="cuda")
        dk = torch.full(k.shape, init, device="cuda")
        dv = torch.full(v.shape, init, device="cuda")
        cp.ring_bwd(q, k, v, d_o, o, lse, delta, dq, dk, dv, 1, True)
        grads.append([t.cpu().numpy() for t in (dq, dk, dv)])
    for a, b in zip(*grads):
        assert np.allclose(b - 1.5, a, atol=1e-5)


def test_backward_is_deterministic():
    wl = small_workload(204, "bf16", 8, 2, 128, 384, 4, True, backward=True)
    a = _ring_fwd_bwd(wl, 3)
    b = _ring_fwd_bwd(wl, 3)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_gradient_invariants_and_constant_v():
    wl = small_workload(205, "bf16", 4, 2, 128, 256, 3, True, backward=True)
    r = 2
    dq, dk, dv = _ring_fwd_bwd(wl, r)
    _, _, _, do = host_inputs(wl, r, with_do=True)
    # sum over all keys of dK is zero; sum over keys of dV equals the group's summed dO
    dk_sum = dk.sum(axis=(0, 2))
    assert np.max(np.abs(dk_sum)) <= 2e-2 * np.max(np.abs(dk)) * np.sqrt(dk.shape[2])
    for g in range(wl.heads_kv):
        ref = do[g * wl.group:(g + 1) * wl.group].sum(axis=(0, 1))
        assert np.max(np.abs(dv[:, g].sum(axis=(0, 1)) - ref)) <= 1e-2 * np.max(np.abs(ref))
    # constant V: O is constant, so dQ and dK vanish up to the rounding of P and dS
    q, k, _, d_o = device_inputs(wl, r, with_do=True)
    v = torch.full(k.shape, 0.5, dtype=torch.bfloat16, device="cuda")
    o = torch.empty(q.shape, device="cuda")
    lse = torch.empty(q.shape[:2], device="cuda")
    cp.ring_fwd(q, k, v, o, lse, r, True)
    delta = torch.empty_like(lse)
    dq0, dk0, dv0 = (torch.zeros_like(o), torch.zeros(k.shape, device="cuda"),
                     torch.zeros(k.shape, device="cuda"))
    cp.ring_bwd(q, k, v, d_o, o, lse, delta, dq0, dk0, dv0, r, True)
    torch.cuda.synchronize()
    assert float(dq0.abs().max()) <= 2e-2 * float(np.max(np.abs(dq)))
    assert float(dk0.abs().max()) <= 2e-2 * float(np.max(np.abs(dk)))


def _wide_grid_workgroups(hq, hkv, lc):
    # 8-wavefront workgroups of one backward launch: one mixed dK/dV workgroup per 128 keys of
    # each key/value head and one dQ workgroup per 256 query rows of each query head; the
    # launch takes 8-wavefront workgroups from 2048 of them up.
    return -(-lc // 128) * hkv + -(-lc // 256) * hq


@pytest.mark.parametrize("d,lc", [(128, 1000), (64, 1000), (128, 1050)])
def test_wide_grid_launch(d, lc):
    """Backward launches large enough for 8-wavefront workgroups (the configuration of the
    208K shard), at a size the full oracle checks: 256 query heads over 128 key/value heads,
    1000- or 1050-row chunks (ragged against the 256-key and 256-row workgroups and the 64-row
    tiles), rank 1 of 2 (one diagonal step, one fully visible step). In the fully visible step
    the last round of dQ work items runs as split workgroups (two groups of four wavefronts on
    the two halves of the keys): 16 key tiles split evenly, 17 leave group B one tile short."""
    hq, hkv = 256, 128
    assert _wide_grid_workgroups(hq, hkv, lc) >= 2048
    wl = small_workload(205, "bf16", hq, hkv, d, lc, 2, True, backward=True)
    r = 1
    dq, dk, dv = _ring_fwd_bwd(wl, r)
    q, k, v, do = host_inputs(wl, r, with_do=True)
    dq_ref, dk_ref, dv_ref = oracle.rank_backward(q, k, v, do, r, True)
    _check_grad(dq, dq_ref, "dQ")
    _check_grad(dk, dk_ref, "dK")
    _check_grad(dv, dv_ref, "dV")


@pytest.mark.parametrize("d,causal", [(128, True), (64, False)])
def test_wide_grid_launch_tiny_rows(d, causal):
    """The 8-wavefront launch reached through the head count alone: 1024 heads of 5-row
    chunks (one 128-key workgroup and one 256-row dQ workgroup per head, almost all of it past
    the end of the chunk)."""
    hq = hkv = 1024
    assert _wide_grid_workgroups(hq, hkv, 5) >= 2048
    wl = small_workload(207, "bf16", hq, hkv, d, 5, 2, causal, backward=True)
    r = 1
    dq, dk, dv = _ring_fwd_bwd(wl, r)
    q, k, v, do = host_inputs(wl, r, with_do=True)
    dq_ref, dk_ref, dv_ref = oracle.rank_backward(q, k, v, do, r, causal)
    _check_grad(dq, dq_ref, "dQ")
    _check_grad(dk, dk_ref, "dK")
    _check_grad(dv, dv_ref, "dV")
