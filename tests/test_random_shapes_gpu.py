"""Single ring steps on seeded random shapes, forward and backward, against the fp64 oracle:
head counts and groupings, both head sizes, lengths from 1 to 400 (ragged against every tile
size), arbitrary global offsets under causality (including steps where some or all rows see
nothing) and non-causal steps. The shapes come from a fixed seed, so every run checks the same
cases."""
import numpy as np
import pytest
import torch

import oracle
from long_context_sequence_amd import binding as cp
from long_context_sequence_amd import inputs

from util import GRAD_REL, check_o_lse

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.integers(1, 5))
        grp = int(rng.integers(1, 5))
        d = int(rng.choice([64, 128]))
        lq, lk = (int(x) for x in rng.integers(1, 401, 2))
        causal = bool(rng.random() < 0.75)
        q0, k0 = (int(x) for x in rng.integers(0, 601, 2)) if causal else (0, 0)
        dtype = "f32" if i % 8 == 7 else "bf16"
        out.append((i, hkv * grp, hkv, d, lq, lk, q0, k0, causal, dtype))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "h{1}-{2}_d{3}_q{4}@{6}_k{5}@{7}_{8}_{9}".format(*c))
def test_random_step_fwd_bwd(case):
    i, hq, hkv, d, lq, lk, q0, k0, causal, dtype = case
    key = 300 + i
    qa = inputs.make(key, "q", 0, (hq, lq, d), dtype)
    ka = inputs.make(key, "k", 0, (hkv, lk, d), dtype)
    va = inputs.make(key, "v", 0, (hkv, lk, d), dtype)
    da = inputs.make(key, "do", 0, (hq, lq, d), dtype)
    q, k, v, d_o = (inputs.to_torch(a, "cuda") for a in (qa, ka, va, da))
    qh, kh, vh, dh = (inputs.widen(a) for a in (qa, ka, va, da))
    o_ref, lse_ref = oracle.attention_forward(qh, kh, vh, q_pos0=q0, kv_pos0=k0, causal=causal)

    o = torch.full(q.shape, 7.0, device="cuda")
    lse = torch.full(q.shape[:2], 7.0, device="cuda")
    st = cp.step(q, k, v, o, lse, q_pos0=q0, kv_pos0=k0, causal=causal)
    torch.cuda.synchronize()
    if st == cp.CP_STEP_SKIPPED:  # no key visible to any row: nothing written
        assert np.all(np.isneginf(lse_ref))
        assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
        return
    check_o_lse(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, dtype, f"case {i}")
    if dtype != "bf16":
        return

    delta = torch.empty_like(lse)
    cp.bwd_prep(o, d_o, delta)
    dq = torch.zeros_like(o)
    dk = torch.zeros(k.shape, device="cuda")
    dv = torch.zeros(v.shape, device="cuda")
    cp.bwd(q, k, v, d_o, lse, delta, dq, dk, dv, q_pos0=q0, kv_pos0=k0, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(qh, kh, vh, dh, q_pos0=q0, kv_pos0=k0, causal=causal)
    for name, got, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        got = got.cpu().numpy()
        scale = float(np.max(np.abs(r)))
        err = float(np.max(np.abs(got - r)))
        assert err <= GRAD_REL * scale + 1e-6, f"case {i} {name}: {err:.3g} vs {scale:.3g}"
    empty = np.isneginf(lse_ref)  # rows that see no key get no gradient
    assert not np.any(dq.cpu().numpy()[empty])


def _wide_cases(n=4, seed=77):
    """Backward steps large enough for the 8-wavefront launch (at least 2,048 workgroups: one
    per 128 keys of each key/value head plus one per 256 rows of each query head), ragged
    lengths, both head sizes; two non-causal steps, one causal step whose keys all precede the
    rows (both take the split dQ tail) and one causal step across the diagonal."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = 128 if i % 2 == 0 else 64
        grp = int(rng.choice([1, 2, 4]))
        hkv = 256 // grp if grp > 1 else 160
        hq = hkv * grp
        lq, lk = (int(x) for x in rng.integers(520, 1100, 2))
        while -(-lk // 128) * hkv + -(-lq // 256) * hq < 2048:
            lk += 128
        causal = i >= 2
        if i == 2:
            q0, k0 = lk + int(rng.integers(0, 300)), 0  # every key visible to every row
        elif i == 3:
            k0 = int(rng.integers(0, 200))
            q0 = k0 + int(rng.integers(0, lk // 2))     # the diagonal crosses the chunk
        else:
            q0 = k0 = 0
        out.append((i, hq, hkv, d, lq, lk, q0, k0, causal))
    return out


@pytest.mark.parametrize("case", _wide_cases(), ids=lambda c: "h{1}-{2}_d{3}_q{4}@{6}_k{5}@{7}_{8}".format(*c))
def test_random_wide_grid_bwd(case):
    i, hq, hkv, d, lq, lk, q0, k0, causal = case
    key = 400 + i
    qa = inputs.make(key, "q", 0, (hq, lq, d), "bf16")
    ka = inputs.make(key, "k", 0, (hkv, lk, d), "bf16")
    va = inputs.make(key, "v", 0, (hkv, lk, d), "bf16")
    da = inputs.make(key, "do", 0, (hq, lq, d), "bf16")
    q, k, v, d_o = (inputs.to_torch(a, "cuda") for a in (qa, ka, va, da))
    qh, kh, vh, dh = (inputs.widen(a) for a in (qa, ka, va, da))
    o = torch.empty(q.shape, device="cuda")
    lse = torch.empty(q.shape[:2], device="cuda")
    cp.step(q, k, v, o, lse, q_pos0=q0, kv_pos0=k0, causal=causal)
    delta = torch.empty_like(lse)
    cp.bwd_prep(o, d_o, delta)
    dq = torch.zeros_like(o)
    dk = torch.zeros(k.shape, device="cuda")
    dv = torch.zeros(v.shape, device="cuda")
    cp.bwd(q, k, v, d_o, lse, delta, dq, dk, dv, q_pos0=q0, kv_pos0=k0, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(qh, kh, vh, dh, q_pos0=q0, kv_pos0=k0, causal=causal)
    for name, got, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        got = got.cpu().numpy()
        scale = float(np.max(np.abs(r)))
        err = float(np.max(np.abs(got - r)))
        assert err <= GRAD_REL * scale + 1e-6, f"wide case {i} {name}: {err:.3g} vs {scale:.3g}"
