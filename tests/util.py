"""Helpers shared by the GPU tests: seeded inputs on the device, the library's ring run, and
the oracle on the same inputs."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
from long_context_sequence_amd import configs, inputs

# Parity bars. bf16 inputs: |dO| <= 2e-2 and |dLSE| <= 1e-3 absolute, plus the same 2e-2 on
# max|dO| / max|O| because |O| shrinks like sqrt(e / n) at long sequences. fp32: 1e-5.
BF16_O_ABS, BF16_O_REL, BF16_LSE_ABS = 2e-2, 2e-2, 1e-3
F32_ABS = 1e-5
GRAD_REL = 5e-2


def small_workload(key, dtype, hq, hkv, d, lc, n_cp, causal, rms=False, backward=False):
    return configs.Workload(key, f"test-{key}", dtype, hq, hkv, d, lc * n_cp, n_cp, causal,
                            tuple(range(n_cp)), rms_rows=rms, backward=backward)


def device_inputs(wl, rank, device="cuda", with_do=False):
    import torch  # noqa: F401

    q = inputs.to_torch(inputs.workload_tensor(wl, "q", rank), device)
    k = inputs.to_torch(inputs.workload_kv(wl, "k"), device)
    v = inputs.to_torch(inputs.workload_kv(wl, "v"), device)
    if with_do:
        return q, k, v, inputs.to_torch(inputs.workload_tensor(wl, "do", rank), device)
    return q, k, v


def host_inputs(wl, rank, with_do=False):
    q = inputs.widen(inputs.workload_tensor(wl, "q", rank))
    k = inputs.widen(inputs.workload_kv(wl, "k"))
    v = inputs.widen(inputs.workload_kv(wl, "v"))
    if with_do:
        return q, k, v, inputs.widen(inputs.workload_tensor(wl, "do", rank))
    return q, k, v


def check_o_lse(o, lse, o_ref, lse_ref, dtype, what=""):
    """Element-wise comparison at the parity bar for the dtype; returns the errors."""
    o, lse, o_ref, lse_ref = (np.asarray(x, dtype=np.float64) for x in (o, lse, o_ref, lse_ref))
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), f"{what}: -inf pattern differs"
    fin = np.isfinite(lse_ref)
    e_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    e_l = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    scale_o = float(np.max(np.abs(o_ref))) if o.size else 1.0
    if dtype == "f32":
        assert e_o <= F32_ABS and e_l <= F32_ABS, f"{what}: fp32 errors O {e_o:.3g} LSE {e_l:.3g}"
    else:
        assert e_o <= BF16_O_ABS, f"{what}: max|dO| {e_o:.3g}"
        assert e_o <= BF16_O_REL * max(scale_o, 1e-30), f"{what}: max|dO|/max|O| {e_o / scale_o:.3g}"
        assert e_l <= BF16_LSE_ABS, f"{what}: max|dLSE| {e_l:.3g}"
    return e_o, e_l


def oracle_rank(wl, rank):
    q, k, v = host_inputs(wl, rank)
    return oracle.rank_forward(q, k, v, rank, wl.causal, scale=wl.scale)


def sample_rows(wl, rank, n, seed):
    """(heads, rows) of n sampled query rows incl. first/last rows of the shard."""
    rng = np.random.default_rng(seed)
    lc = wl.chunk_len
    rows = np.concatenate([[0, 1, lc - 1, lc // 2], rng.integers(0, lc, n - 4)])[:n]
    heads = rng.integers(0, wl.heads_q, n)
    heads[:4] = [0, wl.heads_q - 1, wl.heads_q // 2, 1 % wl.heads_q]
    return heads, rows


def host_workers() -> int:
    """Host cores this process may use (at most 16: one GPU's share of a host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_map(fn, items):
    """fn over items on the host cores: a thread pool with BLAS held to one thread per call.
    numpy releases the GIL inside its array kernels, so the calls run in parallel; threads
    rather than processes, because this process already holds the GPU."""
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(host_workers()) as ex:
            return list(ex.map(fn, items))
