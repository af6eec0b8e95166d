"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test is chosen so that a plausible slip in the oracle (a dropped term, a wrong sign, a
transposed operand, a wrong head map or causal offset, log2 instead of ln) fails at least one:
  * torch's CPU scaled_dot_product_attention in float64 with an explicit boolean mask and
    enable_gqa, and its autograd, as an independent library implementation;
  * closed forms: a single visible key, uniform scores, two keys;
  * invariants: rows sum to one, chunked online-softmax merge equals full attention in any ring
    order (ring attention on the context-parallelism page: the ring reaches full attention),
    gradient sums, constant V;
  * central finite differences of the loss sum(O * dO).
"""
import itertools

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(1234)


def _rand(*shape):
    return RNG.standard_normal(shape)


def _sdpa(q, k, v, mask, scale):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    m = torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        tq[None], tk[None], tv[None], attn_mask=m, scale=scale,
        enable_gqa=tq.shape[0] != tk.shape[0])[0].numpy()


@pytest.mark.parametrize("hq,hkv,lq,lk,d,q0,k0,causal", [
    (2, 2, 7, 9, 8, 0, 0, False),
    (4, 2, 6, 11, 16, 20, 15, True),      # GQA, causal with global offsets, partly masked rows
    (6, 3, 5, 5, 4, 10, 10, True),        # diagonal block
    (4, 1, 3, 12, 8, 100, 0, True),       # MQA, all keys visible
])
def test_forward_matches_torch_sdpa(hq, hkv, lq, lk, d, q0, k0, causal):
    q, k, v = _rand(hq, lq, d), _rand(hkv, lk, d), _rand(hkv, lk, d)
    o, lse = oracle.attention_forward(q, k, v, q_pos0=q0, kv_pos0=k0, causal=causal)
    mask = (k0 + np.arange(lk))[None, :] <= (q0 + np.arange(lq))[:, None] if causal else \
        np.ones((lq, lk), dtype=bool)
    ref = _sdpa(q, k, v, mask, 1.0 / np.sqrt(d))
    assert np.max(np.abs(o - ref)) < 1e-12
    # LSE through a one-hot V: O[i, j] = P_ij = exp(s_ij - LSE_i), with s from torch's matmul.
    eye_v = np.zeros((hkv, lk, lk))
    eye_v[:, np.arange(lk), np.arange(lk)] = 1.0
    p, lse2 = oracle.attention_forward(q, k, eye_v, q_pos0=q0, kv_pos0=k0, causal=causal,
                                       scale=1.0 / np.sqrt(d))
    assert np.max(np.abs(lse - lse2)) == 0.0
    grp = hq // hkv
    tq, tk = torch.from_numpy(q), torch.from_numpy(k)
    for h in range(hq):
        s = (tq[h] @ tk[h // grp].T).numpy() / np.sqrt(d)
        vis = mask
        ref_p = np.exp(s - lse[h][:, None]) * vis
        assert np.max(np.abs(p[h] - ref_p)) < 1e-12
        assert np.allclose(ref_p.sum(axis=1), 1.0, atol=1e-12)   # rows sum to one, natural log


def test_full_causal_sequence_matches_is_causal():
    # Over a whole sequence (Lq = Lk, both from position 0) top-left causal alignment is right.
    h, l, d = 3, 24, 8
    q, k, v = _rand(h, l, d), _rand(h, l, d), _rand(h, l, d)
    o, _ = oracle.attention_forward(q, k, v, causal=True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        is_causal=True)[0].numpy()
    assert np.max(np.abs(o - ref)) < 1e-12


def test_rank_forward_is_a_slice_of_full_sequence_attention():
    hq, hkv, n, lc, d = 4, 2, 4, 6, 8
    kc, vc = _rand(n, hkv, lc, d), _rand(n, hkv, lc, d)
    qfull = _rand(hq, n * lc, d)
    kfull = np.concatenate(list(kc), axis=1)
    vfull = np.concatenate(list(vc), axis=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qfull)[None], torch.from_numpy(kfull)[None],
        torch.from_numpy(vfull)[None], is_causal=True, enable_gqa=True)[0].numpy()
    for r in range(n):
        o, _ = oracle.rank_forward(qfull[:, r * lc:(r + 1) * lc], kc, vc, r, causal=True)
        assert np.max(np.abs(o - ref[:, r * lc:(r + 1) * lc])) < 1e-12


def test_single_visible_key_closed_form():
    hq, lc, d = 2, 5, 16
    q, k, v = _rand(hq, lc, d), _rand(hq, lc, d), _rand(hq, lc, d)
    o, lse = oracle.attention_forward(q, k, v, causal=True)
    for h in range(hq):
        assert np.allclose(o[h, 0], v[h, 0], atol=1e-14)
        assert abs(lse[h, 0] - q[h, 0] @ k[h, 0] / np.sqrt(d)) < 1e-13


def test_uniform_scores_closed_form():
    # q = 0: every visible score is 0, LSE = ln(#visible), O = mean of the visible V rows.
    hq, lq, lk, d = 2, 5, 9, 4
    q = np.zeros((hq, lq, d))
    k, v = _rand(hq, lk, d), _rand(hq, lk, d)
    o, lse = oracle.attention_forward(q, k, v, q_pos0=3, kv_pos0=0, causal=True)
    for i in range(lq):
        nvis = min(lk, 3 + i + 1)
        assert np.allclose(lse[:, i], np.log(nvis), atol=1e-14)
        assert np.allclose(o[:, i], v[:, :nvis].mean(axis=1), atol=1e-14)


def test_two_key_closed_form():
    d = 4
    q = np.array([[[1.0, 0, 0, 0]]])
    k = np.array([[[2.0, 0, 0, 0], [-1.0, 0, 0, 0]]])
    v = np.array([[[1.0, 2, 3, 4], [5.0, 6, 7, 8]]])
    o, lse = oracle.attention_forward(q, k, v, scale=0.5)
    a, b = 1.0, -0.5
    w = np.exp(a) / (np.exp(a) + np.exp(b))
    assert abs(lse[0, 0] - np.log(np.exp(a) + np.exp(b))) < 1e-14
    assert np.allclose(o[0, 0], w * v[0, 0] + (1 - w) * v[0, 1], atol=1e-14)
    assert d == q.shape[-1]


def test_constant_v_gives_constant_output_and_zero_grads():
    hq, hkv, lq, lk, d = 4, 2, 6, 10, 8
    q, k = _rand(hq, lq, d), _rand(hkv, lk, d)
    v = np.full((hkv, lk, d), 0.75)
    o, _ = oracle.attention_forward(q, k, v, q_pos0=4, causal=True)
    assert np.allclose(o, 0.75, atol=1e-14)
    dq, dk, dv = oracle.attention_backward(q, k, v, _rand(hq, lq, d), q_pos0=4, causal=True)
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13


def test_empty_visible_set():
    q, k, v = _rand(1, 3, 4), _rand(1, 2, 4), _rand(1, 2, 4)
    o, lse = oracle.attention_forward(q, k, v, q_pos0=0, kv_pos0=1, causal=True)
    assert np.all(o[0, 0] == 0) and np.isneginf(lse[0, 0])      # row 0 sees nothing
    assert np.isfinite(lse[0, 1:]).all()
    o, lse = oracle.attention_forward(q, k[:, :0], v[:, :0])
    assert np.all(o == 0) and np.isneginf(lse).all()


@pytest.mark.parametrize("causal", [False, True])
def test_chunked_merge_equals_full_attention_in_any_order(causal):
    hq, hkv, n, lc, d = 4, 2, 4, 5, 8
    kc, vc = _rand(n, hkv, lc, d), _rand(n, hkv, lc, d)
    for r in range(n):
        q = _rand(hq, lc, d)
        full_o, full_lse = oracle.rank_forward(q, kc, vc, r, causal)
        parts = [oracle.attention_forward(q, kc[c], vc[c], q_pos0=r * lc, kv_pos0=c * lc,
                                          causal=causal) for c in range(n)]
        for order in itertools.permutations(range(n)):
            o, lse = parts[order[0]]
            for c in order[1:]:
                o, lse = oracle.merge(o, lse, *parts[c])
            assert np.max(np.abs(o - full_o)) < 1e-12
            assert np.max(np.abs(lse - full_lse)) < 1e-12


def test_merge_identity_symmetry_and_empty():
    o, lse = _rand(2, 3, 4), _rand(2, 3)
    empty_o, empty_lse = np.zeros((2, 3, 4)), np.full((2, 3), -np.inf)
    mo, ml = oracle.merge(o, lse, empty_o, empty_lse)
    assert np.array_equal(ml, lse) and np.allclose(mo, o, atol=0)
    mo, ml = oracle.merge(empty_o, empty_lse, empty_o, empty_lse)
    assert np.all(mo == 0) and np.isneginf(ml).all()
    o2, lse2 = _rand(2, 3, 4), _rand(2, 3)
    a = oracle.merge(o, lse, o2, lse2)
    b = oracle.merge(o2, lse2, o, lse)
    assert np.allclose(a[0], b[0], atol=1e-15) and np.allclose(a[1], b[1], atol=1e-15)
    assert np.allclose(a[1], np.logaddexp(lse, lse2), atol=1e-14)


def test_lse_statistics_of_gaussian_scores():
    # q, k ~ N(0, 1) and scale 1/sqrt(d) give scores ~ N(0, 1); E[exp(s)] = e^(1/2), so the
    # mean of LSE - ln(#keys) tends to 1/2 for many keys.
    d, lk = 64, 4096
    q, k, v = _rand(1, 64, d), _rand(1, lk, d), _rand(1, lk, d)
    _, lse = oracle.attention_forward(q, k, v)
    assert abs(np.mean(lse) - np.log(lk) - 0.5) < 0.05


@pytest.mark.parametrize("hq,hkv,lq,lk,q0,k0,causal", [
    (4, 2, 5, 7, 3, 0, True),
    (2, 2, 4, 6, 0, 0, False),
    (4, 1, 6, 6, 6, 6, True),
])
def test_backward_matches_torch_autograd(hq, hkv, lq, lk, q0, k0, causal):
    d = 8
    q, k, v, do = _rand(hq, lq, d), _rand(hkv, lk, d), _rand(hkv, lk, d), _rand(hq, lq, d)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, q_pos0=q0, kv_pos0=k0, causal=causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = torch.from_numpy(oracle.visibility(lq, lk, q0, k0, causal))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq[None], tk[None], tv[None], attn_mask=mask, enable_gqa=hq != hkv)[0]
    (out * torch.from_numpy(do)).sum().backward()
    assert np.max(np.abs(dq - tq.grad.numpy())) < 1e-12
    assert np.max(np.abs(dk - tk.grad.numpy())) < 1e-12
    assert np.max(np.abs(dv - tv.grad.numpy())) < 1e-12


def test_backward_finite_differences():
    hq, hkv, n, lc, d = 4, 2, 4, 4, 8
    rng = np.random.default_rng(7)
    q = rng.standard_normal((hq, lc, d))
    kc, vc = rng.standard_normal((n, hkv, lc, d)), rng.standard_normal((n, hkv, lc, d))
    do = rng.standard_normal((hq, lc, d))
    r = 2
    dq, dk, dv = oracle.rank_backward(q, kc, vc, do, r, causal=True)

    def loss(qq, kk, vv):
        return float(np.sum(oracle.rank_forward(qq, kk, vv, r, causal=True)[0] * do))

    h = 1e-6
    for arr, grad in ((q, dq), (kc, dk), (vc, dv)):
        for idx in [tuple(rng.integers(0, s) for s in arr.shape) for _ in range(12)]:
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += h
            minus[idx] -= h
            args_p = [plus if a is arr else a for a in (q, kc, vc)]
            args_m = [minus if a is arr else a for a in (q, kc, vc)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-7, (idx, fd, grad[idx])
    # chunks after the rank's own are in the future: no gradient flows to them
    assert np.all(dk[r + 1:] == 0) and np.all(dv[r + 1:] == 0)


def test_gradient_invariants_and_softmax_dot():
    hq, hkv, lq, lk, d = 4, 2, 9, 13, 8
    q, k, v, do = _rand(hq, lq, d), _rand(hkv, lk, d), _rand(hkv, lk, d), _rand(hq, lq, d)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, q_pos0=5, causal=True)
    # sum_j dS_ij = 0 for every row, so sum_j dK_j = 0; rows of P sum to 1, so
    # sum_j dV_j = sum over the group's heads and rows of dO.
    assert np.max(np.abs(dk.sum(axis=1))) < 1e-12
    for g in range(hkv):
        ref = do[2 * g:2 * g + 2].sum(axis=(0, 1))
        assert np.max(np.abs(dv[g].sum(axis=0) - ref)) < 1e-12
    o, _ = oracle.attention_forward(q, k, v, q_pos0=5, causal=True)
    assert np.max(np.abs(oracle.softmax_dot(q, k, v, do, q_pos0=5, causal=True)
                         - np.sum(o * do, axis=-1))) < 1e-12


def test_attention_rows_agrees_with_attention_forward():
    hq, hkv, lq, lk, d = 4, 2, 8, 20, 16
    q, k, v = _rand(hq, lq, d), _rand(hkv, lk, d), _rand(hkv, lk, d)
    o, lse = oracle.attention_forward(q, k, v, q_pos0=12, causal=True)
    heads = np.array([0, 3, 1, 2, 3])
    rows = np.array([0, 7, 4, 1, 2])
    o2, lse2 = oracle.attention_rows(q[heads, rows], k, v, heads, rows, hq, q_pos0=12,
                                     causal=True)
    assert np.max(np.abs(o2 - o[heads, rows])) < 1e-13
    assert np.max(np.abs(lse2 - lse[heads, rows])) < 1e-13


def test_attention_backward_rows_agrees_with_attention_backward():
    """The row-restricted backward (used at sizes where the full gradient is out of reach)
    against attention_backward, which autograd and finite differences pin: dQ on any rows;
    dK/dV at chosen keys from exactly the rows that can see them (causal: query position >=
    key position), so the partial sums are complete there."""
    hq, hkv, lq, lk, d = 4, 2, 10, 30, 16
    q, k, v, do = _rand(hq, lq, d), _rand(hkv, lk, d), _rand(hkv, lk, d), _rand(hq, lq, d)
    q0 = 20  # query rows at positions 20..29, keys at 0..29
    dq, dk, dv = oracle.attention_backward(q, k, v, do, q_pos0=q0, causal=True)
    heads = np.array([0, 3, 1, 2, 3, 0])
    rows = np.array([0, 9, 4, 1, 2, 5])
    dq2, _, _ = oracle.attention_backward_rows(q[heads, rows], do[heads, rows], k, v, heads,
                                               rows, hq, q_pos0=q0, causal=True)
    assert np.max(np.abs(dq2 - dq[heads, rows])) < 1e-13
    keys = np.array([25, 29, 27])  # seen by the rows at positions >= 25 only
    hh, rr = np.meshgrid(np.arange(hq), np.arange(5, lq), indexing="ij")
    hh, rr = hh.ravel(), rr.ravel()
    _, dk2, dv2 = oracle.attention_backward_rows(q[hh, rr], do[hh, rr], k, v, hh, rr, hq,
                                                 q_pos0=q0, causal=True, keys=keys)
    assert np.max(np.abs(dk2 - dk[:, keys])) < 1e-13
    assert np.max(np.abs(dv2 - dv[:, keys])) < 1e-13


def test_golden_c1_rank0_fixture():
    import json
    import os

    from long_context_sequence_amd import configs, inputs

    path = os.path.join(os.path.dirname(__file__), "golden", "c1_rank0.json")
    with open(path) as f:
        gold = json.load(f)
    wl = configs.C1
    q = inputs.widen(inputs.workload_tensor(wl, "q", 0))
    k = inputs.widen(inputs.workload_kv(wl, "k"))
    v = inputs.widen(inputs.workload_kv(wl, "v"))
    o, lse = oracle.rank_forward(q, k, v, 0, wl.causal)
    assert np.max(np.abs(lse - np.array(gold["lse"]))) < 1e-12
    assert np.max(np.abs(o[:, gold["rows"]] - np.array(gold["o_rows"]))) < 1e-12
