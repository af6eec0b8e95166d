"""ctypes binding of libcp_attn.so (the C ABI in include/cp_attn.h and include/cp_fir.h).

Argument marshalling only: tensors are checked for device, dtype, shape and contiguity, then
their device pointers and torch's current HIP stream are handed to the library. Every step of
the computation runs in the library's kernels. If the library has not been built this module
raises on first use; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

# The in-tree build; CP_ATTN_LIB may point at another build of the same sources (development).
_LIB_PATH = os.environ.get("CP_ATTN_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libcp_attn.so")

CP_OK, CP_STEP_SKIPPED = 0, 1
CP_F32, CP_BF16 = 0, 1


class CpAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("len_q", ctypes.c_int32), ("len_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("q_pos0", ctypes.c_int64), ("kv_pos0", ctypes.c_int64),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("accumulate", ctypes.c_int32)]


class FirDesc(ctypes.Structure):
    _fields_ = [("channels", ctypes.c_int32), ("shard_len", ctypes.c_int32),
                ("taps", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class RingDesc(ctypes.Structure):
    _fields_ = [("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("chunk_len", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_cp", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libcp_attn.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it first "
                           "(python -m long_context_sequence_amd.build)")
    lib = ctypes.CDLL(_LIB_PATH)
    st = ctypes.c_int32
    lib.cp_attn_step.argtypes = [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P]
    lib.cp_attn_step.restype = st
    lib.cp_attn_merge.argtypes = [ctypes.c_int64, ctypes.c_int32, _P, _P, _P, _P, _P]
    lib.cp_attn_merge.restype = st
    lib.cp_attn_bwd_prep.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P]
    lib.cp_attn_bwd_prep.restype = st
    lib.cp_attn_bwd.argtypes = [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.cp_attn_bwd.restype = st
    lib.cp_attn_bwd_dkdv.argtypes = [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.cp_attn_bwd_dkdv.restype = st
    lib.cp_attn_bwd_dq.argtypes = [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P, _P]
    lib.cp_attn_bwd_dq.restype = st
    lib.cp_ring_schedule.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.cp_ring_schedule.restype = ctypes.c_int32
    lib.cp_attn_ring_fwd.argtypes = [ctypes.POINTER(RingDesc), _P, _P, _P, _P, _P, _P, _P, _P]
    lib.cp_attn_ring_fwd.restype = st
    lib.cp_attn_ring_bwd.argtypes = [ctypes.POINTER(RingDesc), _P, _P, _P, _P, _P, _P, _P, _P,
                                     _P, _P, _P]
    lib.cp_attn_ring_bwd.restype = st
    lib.cp_attn_ring_bwd_noalloc.argtypes = [ctypes.POINTER(RingDesc), _P, _P, _P, _P, _P, _P,
                                             _P, _P, _P, _P]
    lib.cp_attn_ring_bwd_noalloc.restype = st
    lib.cp_zigzag_shards.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    lib.cp_zigzag_shards.restype = ctypes.c_int32
    lib.cp_attn_ring_fwd_zigzag.argtypes = [ctypes.POINTER(RingDesc), _P, _P, _P, _P, _P, _P]
    lib.cp_attn_ring_fwd_zigzag.restype = st
    lib.cp_attn_ring_bwd_zigzag.argtypes = [ctypes.POINTER(RingDesc), _P, _P, _P, _P, _P, _P, _P,
                                            _P, _P, _P, _P]
    lib.cp_attn_ring_bwd_zigzag.restype = st
    lib.cp_attn_ring_fwd_striped.argtypes = [ctypes.POINTER(RingDesc), _P, _P, _P, _P, _P, _P]
    lib.cp_attn_ring_fwd_striped.restype = st
    lib.cp_attn_ring_bwd_striped.argtypes = [ctypes.POINTER(RingDesc), _P, _P, _P, _P, _P, _P,
                                             _P, _P, _P, _P, _P]
    lib.cp_attn_ring_bwd_striped.restype = st
    lib.cp_fir_local.argtypes = [ctypes.POINTER(FirDesc), _P, _P, _P, _P]
    lib.cp_fir_local.restype = st
    lib.cp_fir_pack_halo.argtypes = [ctypes.POINTER(FirDesc), _P, _P, _P]
    lib.cp_fir_pack_halo.restype = st
    lib.cp_fir_halo.argtypes = [ctypes.POINTER(FirDesc), _P, _P, _P, _P]
    lib.cp_fir_halo.restype = st
    lib.cp_fir_ring.argtypes = [ctypes.POINTER(FirDesc), ctypes.c_int32, _P, _P, _P, _P, _P]
    lib.cp_fir_ring.restype = st
    lib.cp_probe_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, _P, _P]
    lib.cp_probe_mfma_bf16.restype = st
    lib.cp_probe_copy.argtypes = [ctypes.c_int64, _P, _P, _P]
    lib.cp_probe_copy.restype = st
    lib.cp_attn_status_string.argtypes = [ctypes.c_int32]
    lib.cp_attn_status_string.restype = ctypes.c_char_p
    lib.cp_attn_abi_version.argtypes = []
    lib.cp_attn_abi_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().cp_attn_status_string(int(status)).decode()


def abi_version() -> int:
    return int(load().cp_attn_abi_version())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t) -> int:
    if t.dtype == torch.bfloat16:
        return CP_BF16
    if t.dtype == torch.float32:
        return CP_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name, shape=None, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check(status: int, what: str, allow_skip=True) -> int:
    if status == CP_OK or (allow_skip and status == CP_STEP_SKIPPED):
        return status
    raise CpAttnError(status, what)


def _desc(q, k, q_pos0, kv_pos0, causal, scale, accumulate):
    hq, lq, d = q.shape
    hkv, lk, _ = k.shape
    return AttnDesc(hq, hkv, lq, lk, d, int(bool(causal)), int(q_pos0), int(kv_pos0),
                    float(scale) if scale else 0.0, _dtype_code(q), int(bool(accumulate)))


def step(q, k, v, o, lse, q_pos0=0, kv_pos0=0, causal=False, scale=None, accumulate=False):
    """cp_attn_step: q [H_q, L_q, d]; k, v [H_kv, L_kv, d]; o [H_q, L_q, d] fp32; lse [H_q, L_q]
    fp32. Returns CP_OK or CP_STEP_SKIPPED."""
    _need(q, "q")
    _need(k, "k", dtype=q.dtype)
    _need(v, "v", shape=k.shape, dtype=q.dtype)
    _need(o, "o", shape=q.shape, dtype=torch.float32)
    _need(lse, "lse", shape=q.shape[:2], dtype=torch.float32)
    d = _desc(q, k, q_pos0, kv_pos0, causal, scale, accumulate)
    return _check(load().cp_attn_step(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                      _ptr(lse), _stream()), "cp_attn_step")


def merge(o_acc, lse_acc, o, lse):
    """cp_attn_merge (in place on o_acc, lse_acc)."""
    _need(o_acc, "o_acc", dtype=torch.float32)
    _need(lse_acc, "lse_acc", shape=o_acc.shape[:-1], dtype=torch.float32)
    _need(o, "o", shape=o_acc.shape, dtype=torch.float32)
    _need(lse, "lse", shape=lse_acc.shape, dtype=torch.float32)
    rows = math.prod(o_acc.shape[:-1])
    return _check(load().cp_attn_merge(rows, o_acc.shape[-1], _ptr(o_acc), _ptr(lse_acc), _ptr(o),
                                       _ptr(lse), _stream()), "cp_attn_merge", allow_skip=False)


def bwd_prep(o, d_o, delta):
    """cp_attn_bwd_prep: delta = rowsum(dO * O)."""
    _need(o, "o", dtype=torch.float32)
    _need(d_o, "d_o", shape=o.shape)
    _need(delta, "delta", shape=o.shape[:-1], dtype=torch.float32)
    rows = math.prod(o.shape[:-1])
    return _check(load().cp_attn_bwd_prep(rows, o.shape[-1], _dtype_code(d_o), _ptr(o), _ptr(d_o),
                                          _ptr(delta), _stream()), "cp_attn_bwd_prep",
                  allow_skip=False)


def _bwd_inputs(q, k, v, d_o, lse, delta):
    _need(q, "q")
    _need(k, "k", dtype=q.dtype)
    _need(v, "v", shape=k.shape, dtype=q.dtype)
    _need(d_o, "d_o", shape=q.shape, dtype=q.dtype)
    _need(lse, "lse", shape=q.shape[:2], dtype=torch.float32)
    _need(delta, "delta", shape=q.shape[:2], dtype=torch.float32)


def bwd(q, k, v, d_o, lse, delta, dq, dk, dv, q_pos0=0, kv_pos0=0, causal=False, scale=None):
    """cp_attn_bwd: dq, dk, dv (fp32) are accumulated."""
    _bwd_inputs(q, k, v, d_o, lse, delta)
    _need(dq, "dq", shape=q.shape, dtype=torch.float32)
    _need(dk, "dk", shape=k.shape, dtype=torch.float32)
    _need(dv, "dv", shape=k.shape, dtype=torch.float32)
    d = _desc(q, k, q_pos0, kv_pos0, causal, scale, False)
    return _check(load().cp_attn_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(d_o),
                                     _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv),
                                     _stream()), "cp_attn_bwd")


def bwd_dkdv(q, k, v, d_o, lse, delta, dk, dv, q_pos0=0, kv_pos0=0, causal=False, scale=None):
    """cp_attn_bwd_dkdv: the dK/dV half of cp_attn_bwd (dk, dv accumulated)."""
    _bwd_inputs(q, k, v, d_o, lse, delta)
    _need(dk, "dk", shape=k.shape, dtype=torch.float32)
    _need(dv, "dv", shape=k.shape, dtype=torch.float32)
    d = _desc(q, k, q_pos0, kv_pos0, causal, scale, False)
    return _check(load().cp_attn_bwd_dkdv(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(d_o),
                                          _ptr(lse), _ptr(delta), _ptr(dk), _ptr(dv), _stream()),
                  "cp_attn_bwd_dkdv")


def bwd_dq(q, k, v, d_o, lse, delta, dq, q_pos0=0, kv_pos0=0, causal=False, scale=None):
    """cp_attn_bwd_dq: the dQ half of cp_attn_bwd (dq accumulated)."""
    _bwd_inputs(q, k, v, d_o, lse, delta)
    _need(dq, "dq", shape=q.shape, dtype=torch.float32)
    d = _desc(q, k, q_pos0, kv_pos0, causal, scale, False)
    return _check(load().cp_attn_bwd_dq(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(d_o),
                                        _ptr(lse), _ptr(delta), _ptr(dq), _stream()),
                  "cp_attn_bwd_dq")


def ring_schedule(n_cp: int, rank: int, causal: bool):
    """cp_ring_schedule: [(chunk, class)] for the n_cp steps (host only, no GPU needed)."""
    chunks = (ctypes.c_int32 * max(n_cp, 1))()
    classes = (ctypes.c_int32 * max(n_cp, 1))()
    n = load().cp_ring_schedule(int(n_cp), int(rank), int(bool(causal)), chunks, classes)
    if n < 0:
        raise CpAttnError(n, "cp_ring_schedule")
    return [(chunks[s], classes[s]) for s in range(n_cp)]


def _ring(q, k_chunks, rank, causal, scale):
    hq, lc, d = q.shape
    n_cp, hkv = k_chunks.shape[0], k_chunks.shape[1]
    return RingDesc(hq, hkv, lc, d, n_cp, int(rank), int(bool(causal)),
                    float(scale) if scale else 0.0, _dtype_code(q))


def ring_fwd(q, k_chunks, v_chunks, o, lse, rank, causal, scale=None, o_work=None, lse_work=None):
    """cp_attn_ring_fwd: q [H_q, L_c, d]; k_chunks, v_chunks [N_cp, H_kv, L_c, d]."""
    _need(q, "q")
    n_cp, hkv, lc, d = k_chunks.shape
    _need(k_chunks, "k_chunks", shape=(n_cp, hkv, q.shape[1], q.shape[2]), dtype=q.dtype)
    _need(v_chunks, "v_chunks", shape=k_chunks.shape, dtype=q.dtype)
    _need(o, "o", shape=q.shape, dtype=torch.float32)
    _need(lse, "lse", shape=q.shape[:2], dtype=torch.float32)
    if o_work is not None:
        _need(o_work, "o_work", shape=q.shape, dtype=torch.float32)
        _need(lse_work, "lse_work", shape=q.shape[:2], dtype=torch.float32)
    r = _ring(q, k_chunks, rank, causal, scale)
    return _check(load().cp_attn_ring_fwd(ctypes.byref(r), _ptr(q), _ptr(k_chunks), _ptr(v_chunks),
                                          _ptr(o), _ptr(lse), _ptr(o_work), _ptr(lse_work),
                                          _stream()), "cp_attn_ring_fwd", allow_skip=False)


def ring_bwd(q, k_chunks, v_chunks, d_o, o, lse, delta_work, dq, dk_chunks, dv_chunks, rank,
             causal, scale=None):
    """cp_attn_ring_bwd: dq, dk_chunks, dv_chunks (fp32) are accumulated."""
    _need(q, "q")
    _need(k_chunks, "k_chunks", dtype=q.dtype)
    _need(v_chunks, "v_chunks", shape=k_chunks.shape, dtype=q.dtype)
    _need(d_o, "d_o", shape=q.shape, dtype=q.dtype)
    _need(o, "o", shape=q.shape, dtype=torch.float32)
    _need(lse, "lse", shape=q.shape[:2], dtype=torch.float32)
    _need(delta_work, "delta_work", shape=q.shape[:2], dtype=torch.float32)
    _need(dq, "dq", shape=q.shape, dtype=torch.float32)
    _need(dk_chunks, "dk_chunks", shape=k_chunks.shape, dtype=torch.float32)
    _need(dv_chunks, "dv_chunks", shape=k_chunks.shape, dtype=torch.float32)
    r = _ring(q, k_chunks, rank, causal, scale)
    return _check(load().cp_attn_ring_bwd(ctypes.byref(r), _ptr(q), _ptr(k_chunks), _ptr(v_chunks),
                                          _ptr(d_o), _ptr(o), _ptr(lse), _ptr(delta_work), _ptr(dq),
                                          _ptr(dk_chunks), _ptr(dv_chunks), _stream()),
                  "cp_attn_ring_bwd", allow_skip=False)


def ring_bwd_noalloc(q, k_chunks, v_chunks, d_o, o, lse, dq, dk_chunks, dv_chunks, rank,
                     causal, scale=None):
    """cp_attn_ring_bwd_noalloc: cp_attn_ring_bwd with the library's fixed delta scratch."""
    _need(q, "q")
    _need(k_chunks, "k_chunks", dtype=q.dtype)
    _need(v_chunks, "v_chunks", shape=k_chunks.shape, dtype=q.dtype)
    _need(d_o, "d_o", shape=q.shape, dtype=q.dtype)
    _need(o, "o", shape=q.shape, dtype=torch.float32)
    _need(lse, "lse", shape=q.shape[:2], dtype=torch.float32)
    _need(dq, "dq", shape=q.shape, dtype=torch.float32)
    _need(dk_chunks, "dk_chunks", shape=k_chunks.shape, dtype=torch.float32)
    _need(dv_chunks, "dv_chunks", shape=k_chunks.shape, dtype=torch.float32)
    r = _ring(q, k_chunks, rank, causal, scale)
    return _check(load().cp_attn_ring_bwd_noalloc(ctypes.byref(r), _ptr(q), _ptr(k_chunks),
                                                  _ptr(v_chunks), _ptr(d_o), _ptr(o), _ptr(lse),
                                                  _ptr(dq), _ptr(dk_chunks), _ptr(dv_chunks),
                                                  _stream()),
                  "cp_attn_ring_bwd_noalloc", allow_skip=False)


def zigzag_shards(n_cp: int, rank: int):
    """cp_zigzag_shards: the two half-chunk indices a rank holds (host only)."""
    out = (ctypes.c_int32 * 2)()
    st = load().cp_zigzag_shards(int(n_cp), int(rank), out)
    if st < 0:
        raise CpAttnError(st, "cp_zigzag_shards")
    return int(out[0]), int(out[1])


def _ring_zz(q, k_chunks, rank, causal, scale):
    _, hq, lh, d = q.shape
    n_cp, _, hkv = k_chunks.shape[:3]
    return RingDesc(hq, hkv, lh, d, n_cp, int(rank), int(bool(causal)),
                    float(scale) if scale else 0.0, _dtype_code(q))


def ring_fwd_zigzag(q, k_chunks, v_chunks, o, lse, rank, causal, scale=None):
    """cp_attn_ring_fwd_zigzag: q [2, H_q, Lh, d]; k_chunks, v_chunks [N_cp, 2, H_kv, Lh, d];
    o [2, H_q, Lh, d] fp32; lse [2, H_q, Lh] fp32 (half-major layout)."""
    _need(q, "q")
    if q.dim() != 4 or q.shape[0] != 2:
        raise ValueError("q must be [2, H_q, Lh, d]")
    n_cp = k_chunks.shape[0]
    _need(k_chunks, "k_chunks", shape=(n_cp, 2, k_chunks.shape[2], q.shape[2], q.shape[3]),
          dtype=q.dtype)
    _need(v_chunks, "v_chunks", shape=k_chunks.shape, dtype=q.dtype)
    _need(o, "o", shape=q.shape, dtype=torch.float32)
    _need(lse, "lse", shape=q.shape[:3], dtype=torch.float32)
    r = _ring_zz(q, k_chunks, rank, causal, scale)
    return _check(load().cp_attn_ring_fwd_zigzag(ctypes.byref(r), _ptr(q), _ptr(k_chunks),
                                                 _ptr(v_chunks), _ptr(o), _ptr(lse), _stream()),
                  "cp_attn_ring_fwd_zigzag", allow_skip=False)


def ring_bwd_zigzag(q, k_chunks, v_chunks, d_o, o, lse, delta_work, dq, dk_chunks, dv_chunks,
                    rank, causal, scale=None):
    """cp_attn_ring_bwd_zigzag (half-major layout); dq, dk_chunks, dv_chunks accumulated."""
    _need(q, "q")
    _need(k_chunks, "k_chunks", dtype=q.dtype)
    _need(v_chunks, "v_chunks", shape=k_chunks.shape, dtype=q.dtype)
    _need(d_o, "d_o", shape=q.shape, dtype=q.dtype)
    _need(o, "o", shape=q.shape, dtype=torch.float32)
    _need(lse, "lse", shape=q.shape[:3], dtype=torch.float32)
    _need(delta_work, "delta_work", shape=q.shape[:3], dtype=torch.float32)
    _need(dq, "dq", shape=q.shape, dtype=torch.float32)
    _need(dk_chunks, "dk_chunks", shape=k_chunks.shape, dtype=torch.float32)
    _need(dv_chunks, "dv_chunks", shape=k_chunks.shape, dtype=torch.float32)
    r = _ring_zz(q, k_chunks, rank, causal, scale)
    return _check(load().cp_attn_ring_bwd_zigzag(ctypes.byref(r), _ptr(q), _ptr(k_chunks),
                                                 _ptr(v_chunks), _ptr(d_o), _ptr(o), _ptr(lse),
                                                 _ptr(delta_work), _ptr(dq), _ptr(dk_chunks),
                                                 _ptr(dv_chunks), _stream()),
                  "cp_attn_ring_bwd_zigzag", allow_skip=False)


def ring_fwd_striped(q, k_chunks, v_chunks, o, lse, rank, causal, scale=None):
    """cp_attn_ring_fwd_striped: token t on rank t mod N_cp; shapes as ring_fwd (stripes)."""
    _need(q, "q")
    n_cp, hkv, ls, d = k_chunks.shape
    _need(k_chunks, "k_chunks", shape=(n_cp, hkv, q.shape[1], q.shape[2]), dtype=q.dtype)
    _need(v_chunks, "v_chunks", shape=k_chunks.shape, dtype=q.dtype)
    _need(o, "o", shape=q.shape, dtype=torch.float32)
    _need(lse, "lse", shape=q.shape[:2], dtype=torch.float32)
    r = _ring(q, k_chunks, rank, causal, scale)
    return _check(load().cp_attn_ring_fwd_striped(ctypes.byref(r), _ptr(q), _ptr(k_chunks),
                                                  _ptr(v_chunks), _ptr(o), _ptr(lse), _stream()),
                  "cp_attn_ring_fwd_striped", allow_skip=False)


def ring_bwd_striped(q, k_chunks, v_chunks, d_o, o, lse, delta_work, dq, dk_chunks, dv_chunks,
                     rank, causal, scale=None):
    """cp_attn_ring_bwd_striped; dq, dk_chunks, dv_chunks accumulated."""
    _bwd_inputs(q, k_chunks[0], v_chunks[0], d_o, lse, delta_work)
    _need(o, "o", shape=q.shape, dtype=torch.float32)
    _need(dq, "dq", shape=q.shape, dtype=torch.float32)
    _need(dk_chunks, "dk_chunks", shape=k_chunks.shape, dtype=torch.float32)
    _need(dv_chunks, "dv_chunks", shape=k_chunks.shape, dtype=torch.float32)
    r = _ring(q, k_chunks, rank, causal, scale)
    return _check(load().cp_attn_ring_bwd_striped(ctypes.byref(r), _ptr(q), _ptr(k_chunks),
                                                  _ptr(v_chunks), _ptr(d_o), _ptr(o), _ptr(lse),
                                                  _ptr(delta_work), _ptr(dq), _ptr(dk_chunks),
                                                  _ptr(dv_chunks), _stream()),
                  "cp_attn_ring_bwd_striped", allow_skip=False)


# ---- causal FIR convolution (include/cp_fir.h)

def _fir_desc(x, h):
    channels, shard_len = x.shape[-2], x.shape[-1]
    return FirDesc(channels, shard_len, h.shape[1], _dtype_code(x))


def fir_local(x, h, y):
    """cp_fir_local: y [D, Lc] fp32 = zero-history causal convolution of x [D, Lc] with
    h [D, l_h] (same dtype as x)."""
    _need(x, "x")
    _need(h, "h", dtype=x.dtype)
    _need(y, "y", shape=x.shape, dtype=torch.float32)
    if h.dim() != 2 or h.shape[0] != x.shape[0]:
        raise ValueError("h must be [channels, taps]")
    d = _fir_desc(x, h)
    return _check(load().cp_fir_local(ctypes.byref(d), _ptr(x), _ptr(h), _ptr(y), _stream()),
                  "cp_fir_local", allow_skip=False)


def fir_pack_halo(x, taps, halo):
    """cp_fir_pack_halo: halo [D, taps - 1] = the last taps - 1 samples of x [D, Lc]."""
    _need(x, "x")
    _need(halo, "halo", shape=(x.shape[0], taps - 1), dtype=x.dtype)
    d = FirDesc(x.shape[0], x.shape[1], int(taps), _dtype_code(x))
    return _check(load().cp_fir_pack_halo(ctypes.byref(d), _ptr(x), _ptr(halo), _stream()),
                  "cp_fir_pack_halo", allow_skip=False)


def fir_halo(halo, h, y):
    """cp_fir_halo: y[:, :taps - 1] += boundary terms of the previous shard's tail."""
    _need(h, "h")
    _need(halo, "halo", shape=(h.shape[0], h.shape[1] - 1), dtype=h.dtype)
    _need(y, "y", dtype=torch.float32)
    d = FirDesc(y.shape[0], y.shape[1], h.shape[1], _dtype_code(h))
    return _check(load().cp_fir_halo(ctypes.byref(d), _ptr(halo), _ptr(h), _ptr(y), _stream()),
                  "cp_fir_halo", allow_skip=False)


def fir_ring(x_shards, h, halo_work, y_shards):
    """cp_fir_ring over x_shards [N_cp, D, Lc]; y_shards [N_cp, D, Lc] fp32; halo_work
    [N_cp, D, taps - 1] scratch in x's dtype (None allowed when taps == 1)."""
    _need(x_shards, "x_shards")
    n_cp, channels, lc = x_shards.shape
    _need(h, "h", dtype=x_shards.dtype)
    _need(y_shards, "y_shards", shape=x_shards.shape, dtype=torch.float32)
    if halo_work is not None:
        _need(halo_work, "halo_work", shape=(n_cp, channels, h.shape[1] - 1), dtype=x_shards.dtype)
    d = _fir_desc(x_shards, h)
    return _check(load().cp_fir_ring(ctypes.byref(d), n_cp, _ptr(x_shards), _ptr(h),
                                     _ptr(halo_work), _ptr(y_shards), _stream()),
                  "cp_fir_ring", allow_skip=False)


def probe_mfma_bf16(workgroups, iters, sink):
    """cp_probe_mfma_bf16: enqueue the matrix-core rate probe on the current stream; sink is a
    float32 device tensor of at least workgroups * 256 elements. Returns the flops it issues."""
    _need(sink, "sink", dtype=torch.float32)
    if sink.numel() < workgroups * 256:
        raise ValueError("sink must hold workgroups * 256 floats")
    _check(load().cp_probe_mfma_bf16(int(workgroups), int(iters), _ptr(sink), _stream()),
           "cp_probe_mfma_bf16", allow_skip=False)
    return float(workgroups) * 4 * iters * 4 * 32768


def probe_copy(src, dst):
    """cp_probe_copy: dst <- src (float32 device tensors of equal size, a multiple of 4
    elements) on the current stream. Returns the bytes moved (read + written)."""
    _need(src, "src", dtype=torch.float32)
    _need(dst, "dst", shape=src.shape, dtype=torch.float32)
    if src.numel() % 4:
        raise ValueError("the probe copies whole 16-byte elements")
    n4 = src.numel() // 4
    _check(load().cp_probe_copy(n4, _ptr(src), _ptr(dst), _stream()), "cp_probe_copy",
           allow_skip=False)
    return 32.0 * n4
