"""Seeded synthetic inputs shared by the GPU path, the oracle-based tests and the benchmark.

This module holds no attention arithmetic. It draws N(0, 1) tensors with numpy's PCG64,
optionally RMS-normalises each length-d row, and rounds to bfloat16 with round-to-nearest-even.

Seeding: ``SeedSequence([workload_key, tensor_id, index])`` with tensor ids q=1, k=2, v=3, do=4
(attention) and x=5, h=6 (convolution: the signal shards and the filter bank).
``index`` is the rank for the query-side tensors (q, do: [H_q, L_c, d]) and the chunk for the
key/value tensors (k, v: [H_kv, L_c, d]), so every rank sees the same chunks.

Storage forms: float32 arrays for "f32" workloads; uint16 arrays of bfloat16 bit patterns for
"bf16" workloads. ``widen`` turns either into float64 exactly.
"""
from __future__ import annotations

import numpy as np

TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "do": 4, "x": 5, "h": 6}
RMS_EPS = 1e-6


def normal_f32(key: int, tensor: str, index: int, shape) -> np.ndarray:
    ss = np.random.SeedSequence([int(key), TENSOR_IDS[tensor], int(index)])
    gen = np.random.Generator(np.random.PCG64(ss))
    return gen.standard_normal(size=tuple(shape), dtype=np.float32)


def rms_rows(x: np.ndarray) -> np.ndarray:
    """x / sqrt(mean(x^2) + 1e-6) along the last axis, in float32, no learned gain."""
    x = np.asarray(x, dtype=np.float32)
    ms = np.mean(np.square(x, dtype=np.float32), axis=-1, keepdims=True, dtype=np.float32)
    return (x / np.sqrt(ms + np.float32(RMS_EPS))).astype(np.float32)


def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the uint16 bits.

    Inputs here are finite; NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = u + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def widen(arr: np.ndarray) -> np.ndarray:
    """Exact float64 value of a storage-form array (float32 or bf16 bits)."""
    if arr.dtype == np.uint16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def make(key: int, tensor: str, index: int, shape, dtype: str, rms: bool = False) -> np.ndarray:
    x = normal_f32(key, tensor, index, shape)
    if rms and tensor in ("q", "k", "v"):
        x = rms_rows(x)
    if dtype == "bf16":
        return bf16_rne_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def shard_shape(wl, tensor: str):
    heads = wl.heads_q if tensor in ("q", "do") else wl.heads_kv
    return (heads, wl.chunk_len, wl.head_dim)


def workload_tensor(wl, tensor: str, index: int) -> np.ndarray:
    """One shard (q/do of a rank) or one chunk (k/v) of a workload, in storage form."""
    return make(wl.key, tensor, index, shard_shape(wl, tensor), wl.dtype, rms=wl.rms_rows)


def workload_kv(wl, tensor: str, chunks=None) -> np.ndarray:
    """All (or the listed) K or V chunks stacked as [n_chunks, H_kv, L_c, d]."""
    if chunks is None:
        chunks = range(wl.n_cp)
    return np.stack([workload_tensor(wl, tensor, c) for c in chunks])


def to_torch(arr: np.ndarray, device="cpu"):
    """Storage-form array -> torch tensor (bfloat16 for bit arrays, float32 otherwise)."""
    import torch

    if arr.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def fir_shard(key: int, index: int, channels: int, shard_len: int, dtype: str) -> np.ndarray:
    """Signal shard `index` [D, Lc] of a convolution workload: x ~ N(0, 1)."""
    x = normal_f32(key, "x", index, (channels, shard_len))
    return _store(x, dtype)


def fir_filters(key: int, channels: int, taps: int, dtype: str) -> np.ndarray:
    """Filter bank h [D, l_h]: taps ~ N(0, 1/l_h), so the output stays of order one."""
    h = normal_f32(key, "h", 0, (channels, taps)) * np.float32(1.0 / np.sqrt(taps))
    return _store(h.astype(np.float32), dtype)


def fir_inputs(key: int, n_cp: int, channels: int, shard_len: int, taps: int, dtype: str):
    """All signal shards x [N_cp, D, Lc] (shard r drawn with index r) and the filters h."""
    x = np.stack([fir_shard(key, r, channels, shard_len, dtype) for r in range(n_cp)])
    return x, fir_filters(key, channels, taps, dtype)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_rne_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")
