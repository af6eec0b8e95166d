"""The allocation-free backward ring (cp_attn_ring_bwd_noalloc) against cp_attn_ring_bwd with a
caller-provided delta workspace, through the C ABI: same gradients on two calls in a row, the
second on a smaller input (the fixed scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from long_context_sequence_amd import binding as cp

from util import GRAD_REL, device_inputs, small_workload

pytestmark = pytest.mark.gpu


def _grads(wl, r, noalloc):
    q, k, v, d_o = device_inputs(wl, r, with_do=True)
    o = torch.empty(q.shape, device="cuda")
    lse = torch.empty(q.shape[:2], device="cuda")
    cp.ring_fwd(q, k, v, o, lse, r, wl.causal)
    dq = torch.zeros_like(o)
    dk = torch.zeros(k.shape, device="cuda")
    dv = torch.zeros(v.shape, device="cuda")
    if noalloc:
        cp.ring_bwd_noalloc(q, k, v, d_o, o, lse, dq, dk, dv, r, wl.causal)
    else:
        delta = torch.empty_like(lse)
        cp.ring_bwd(q, k, v, d_o, o, lse, delta, dq, dk, dv, r, wl.causal)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (dq, dk, dv)]


def test_noalloc_matches_workspace_ring_twice_then_smaller():
    big = small_workload(301, "bf16", 8, 2, 128, 520, 3, True, backward=True)
    small = small_workload(302, "bf16", 4, 2, 64, 136, 2, True, backward=True)
    for wl, r in ((big, 2), (small, 1)):
        ref = _grads(wl, r, noalloc=False)
        got = _grads(wl, r, noalloc=True)
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            err = float(np.max(np.abs(a - b)))
            assert err <= GRAD_REL * float(np.max(np.abs(b))), (wl.name, name, err)
            # same kernels on the same inputs: in fact identical
            assert np.array_equal(a, b), (wl.name, name, err)
