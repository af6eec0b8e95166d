"""The C ABI from plain C++ (tests/c_abi_ring.cpp, no Python or torch in the process): one rank's
ring forward and backward on buffers the program allocates itself, checked against the fp64
oracle on the same seeded inputs."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from long_context_sequence_amd import build as lib_build
from long_context_sequence_amd import inputs

from util import GRAD_REL, check_o_lse, small_workload

pytestmark = pytest.mark.gpu


@pytest.mark.skipif(not os.path.exists(lib_build.ABI_EXAMPLE),
                    reason="the C++ ABI consumer is not built (long_context_sequence_amd.build)")
@pytest.mark.parametrize("causal", [True, False])
def test_c_program_ring_fwd_bwd(tmp_path, causal):
    wl = small_workload(210, "bf16", 4, 2, 128, 96, 3, causal, backward=True)
    r = 2
    qa = inputs.workload_tensor(wl, "q", r)
    da = inputs.workload_tensor(wl, "do", r)
    ka, va = inputs.workload_kv(wl, "k"), inputs.workload_kv(wl, "v")
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        np.array([wl.heads_q, wl.heads_kv, wl.chunk_len, wl.head_dim, wl.n_cp, r, int(causal)],
                 dtype=np.int32).tofile(f)
        for a in (qa, ka, va, da):
            np.ascontiguousarray(a, dtype=np.uint16).tofile(f)
    res = subprocess.run([lib_build.ABI_EXAMPLE, str(src), str(dst)], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    out = np.fromfile(dst, dtype=np.float32)
    nq, nrow, nkv = qa.size, qa.shape[0] * qa.shape[1], ka.size
    o, lse, dq, dk, dv = np.split(out, np.cumsum([nq, nrow, nq, nkv]))
    assert dv.size == nkv
    q, k, v, do = (inputs.widen(a) for a in (qa, ka, va, da))
    o_ref, lse_ref = oracle.rank_forward(q, k, v, r, causal)
    check_o_lse(o.reshape(qa.shape), lse.reshape(qa.shape[:2]), o_ref, lse_ref, "bf16", "C ABI")
    refs = oracle.rank_backward(q, k, v, do, r, causal)
    for name, got, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs):
        got = got.reshape(ref.shape)
        err = float(np.max(np.abs(got - ref)))
        assert err <= GRAD_REL * float(np.max(np.abs(ref))), f"{name}: {err:.3g}"
