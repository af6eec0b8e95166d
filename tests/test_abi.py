"""The C ABI without a GPU: the library loads, exports every function include/cp_attn.h
declares, and its host-side validation and ring schedule behave as documented. Only calls that
return before any launch are made here."""
import ctypes
import os
import re

import pytest

from long_context_sequence_amd import binding as cp
from long_context_sequence_amd import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in ("cp_attn.h", "cp_fir.h", "cp_probe.h")]

CP_ERR_NULL, CP_ERR_SHAPE, CP_ERR_DTYPE, CP_ERR_ALIGN, CP_ERR_UNSUPPORTED = -1, -2, -3, -4, -5

needs_lib = pytest.mark.skipif(not os.path.exists(cp.lib_path()),
                               reason="libcp_attn.so not built")


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cp_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("cp_attn_step", "cp_attn_merge", "cp_attn_bwd", "cp_attn_bwd_prep",
                     "cp_ring_schedule", "cp_attn_ring_fwd", "cp_attn_ring_bwd",
                     "cp_attn_status_string", "cp_attn_abi_version", "cp_fir_local",
                     "cp_fir_pack_halo", "cp_fir_halo", "cp_fir_ring", "cp_probe_mfma_bf16", "cp_probe_copy"):
        assert required in names


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(cp.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


@needs_lib
def test_status_strings_and_version():
    assert cp.abi_version() == 1
    for st in range(-7, 2):
        s = cp.status_string(st)
        assert s and s != "unknown status"
    assert cp.status_string(99) == "unknown status"


def _desc(**kw):
    base = dict(heads_q=4, heads_kv=2, len_q=64, len_kv=64, head_dim=128, causal=1, q_pos0=0,
                kv_pos0=0, scale=0.0, dtype=cp.CP_BF16, accumulate=0)
    base.update(kw)
    return cp.AttnDesc(**base)


FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10008)


def _step(d, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE):
    return cp.load().cp_attn_step(ctypes.byref(d) if d is not None else None, q, k, v, o, lse, None)


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(heads_q=3, heads_kv=2), CP_ERR_SHAPE),
    (dict(heads_q=0), CP_ERR_SHAPE),
    (dict(len_q=-1), CP_ERR_SHAPE),
    (dict(len_kv=(1 << 23) + 1), CP_ERR_SHAPE),
    (dict(head_dim=96), CP_ERR_UNSUPPORTED),
    (dict(head_dim=0), CP_ERR_SHAPE),
    (dict(causal=2), CP_ERR_SHAPE),
    (dict(dtype=7), CP_ERR_DTYPE),
    (dict(accumulate=3), CP_ERR_SHAPE),
    (dict(scale=float("nan")), CP_ERR_SHAPE),
])
def test_step_rejects_bad_descriptors(kw, status):
    assert _step(_desc(**kw)) == status


@needs_lib
def test_step_pointer_checks_and_trivial_cases():
    assert _step(None) == CP_ERR_NULL
    assert _step(_desc(), q=None) == CP_ERR_NULL
    assert _step(_desc(), v=MISALIGNED) == CP_ERR_ALIGN
    assert _step(_desc(len_q=0), q=None, k=None, v=None, o=None, lse=None) == 0
    # causal and the chunk starts after the last query: skipped before any pointer is used
    assert _step(_desc(q_pos0=0, kv_pos0=64), q=None) == cp.CP_STEP_SKIPPED
    assert _step(_desc(len_kv=0, accumulate=1), k=None, v=None) == 0


@needs_lib
def test_other_entry_points_validate_first():
    lib = cp.load()
    assert lib.cp_attn_merge(-1, 128, FAKE, FAKE, FAKE, FAKE, None) == CP_ERR_SHAPE
    assert lib.cp_attn_merge(10, 80, FAKE, FAKE, FAKE, FAKE, None) == CP_ERR_UNSUPPORTED
    assert lib.cp_attn_merge(10, 128, FAKE, None, FAKE, FAKE, None) == CP_ERR_NULL
    assert lib.cp_attn_merge(0, 128, None, None, None, None, None) == 0
    assert lib.cp_attn_bwd_prep(10, 128, 5, FAKE, FAKE, FAKE, None) == CP_ERR_DTYPE
    assert lib.cp_attn_bwd_prep(10, 128, 1, MISALIGNED, FAKE, FAKE, None) == CP_ERR_ALIGN
    d = _desc(dtype=cp.CP_F32)
    assert lib.cp_attn_bwd(ctypes.byref(d), *([FAKE] * 9), None) == CP_ERR_UNSUPPORTED
    d = _desc(q_pos0=0, kv_pos0=1000)
    assert lib.cp_attn_bwd(ctypes.byref(d), *([FAKE] * 9), None) == cp.CP_STEP_SKIPPED
    r = cp.RingDesc(4, 2, 64, 128, 4, 4, 1, 0.0, cp.CP_BF16)   # rank out of range
    assert lib.cp_attn_ring_fwd(ctypes.byref(r), *([FAKE] * 5), None, None, None) == CP_ERR_SHAPE
    r = cp.RingDesc(4, 2, 64, 128, 4, 1, 1, 0.0, cp.CP_BF16)
    assert lib.cp_attn_ring_fwd(ctypes.byref(r), *([FAKE] * 5), FAKE, None, None) == CP_ERR_NULL
    assert lib.cp_attn_ring_fwd(ctypes.byref(r), FAKE, FAKE, MISALIGNED, FAKE, FAKE,
                                None, None, None) == CP_ERR_ALIGN


@needs_lib
@pytest.mark.parametrize("n_cp", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_native_ring_schedule_matches_reading(n_cp, causal):
    for r in range(n_cp):
        assert cp.ring_schedule(n_cp, r, causal) == configs.ring_schedule(n_cp, r, causal)


@needs_lib
def test_ring_schedule_errors():
    lib = cp.load()
    buf = (ctypes.c_int32 * 4)()
    assert lib.cp_ring_schedule(0, 0, 0, buf, buf) == CP_ERR_SHAPE
    assert lib.cp_ring_schedule(4, -1, 0, buf, buf) == CP_ERR_SHAPE
    assert lib.cp_ring_schedule(4, 0, 0, None, buf) == CP_ERR_NULL
    assert lib.cp_ring_schedule(4, 3, 1, buf, buf) == 4
    assert lib.cp_ring_schedule(4, 0, 1, buf, buf) == 1


@needs_lib
def test_fir_entry_points_validate_first():
    lib = cp.load()
    ok = cp.FirDesc(4, 64, 5, cp.CP_BF16)
    assert lib.cp_fir_local(None, FAKE, FAKE, FAKE, None) == CP_ERR_NULL
    for bad, status in ((cp.FirDesc(0, 64, 5, 1), CP_ERR_SHAPE), (cp.FirDesc(4, -1, 5, 1), CP_ERR_SHAPE),
                        (cp.FirDesc(4, 64, 0, 1), CP_ERR_SHAPE), (cp.FirDesc(4, 64, 1025, 1), CP_ERR_SHAPE),
                        (cp.FirDesc(4, 3, 5, 1), CP_ERR_SHAPE),     # halo longer than a shard
                        (cp.FirDesc(4, 64, 5, 9), CP_ERR_DTYPE)):
        assert lib.cp_fir_local(ctypes.byref(bad), FAKE, FAKE, FAKE, None) == status
    assert lib.cp_fir_local(ctypes.byref(ok), FAKE, None, FAKE, None) == CP_ERR_NULL
    assert lib.cp_fir_local(ctypes.byref(ok), FAKE, MISALIGNED, FAKE, None) == CP_ERR_ALIGN
    assert lib.cp_fir_local(ctypes.byref(cp.FirDesc(4, 0, 1, 1)), None, None, None, None) == 0
    assert lib.cp_fir_pack_halo(ctypes.byref(cp.FirDesc(4, 64, 1, 1)), None, None, None) == 0
    assert lib.cp_fir_halo(ctypes.byref(ok), FAKE, FAKE, None, None) == CP_ERR_NULL
    assert lib.cp_fir_ring(ctypes.byref(ok), 0, FAKE, FAKE, FAKE, FAKE, None) == CP_ERR_SHAPE
    assert lib.cp_fir_ring(ctypes.byref(ok), 2, FAKE, FAKE, None, FAKE, None) == CP_ERR_NULL


@needs_lib
def test_probe_validation():
    lib = cp.load()
    assert lib.cp_probe_mfma_bf16(4, 10, None, None) == CP_ERR_NULL
    assert lib.cp_probe_mfma_bf16(0, 10, FAKE, None) == CP_ERR_SHAPE
    assert lib.cp_probe_mfma_bf16(4, 0, FAKE, None) == CP_ERR_SHAPE
    assert lib.cp_probe_mfma_bf16((1 << 20) + 1, 10, FAKE, None) == CP_ERR_SHAPE
    assert lib.cp_probe_copy(16, None, FAKE, None) == CP_ERR_NULL
    assert lib.cp_probe_copy(16, ctypes.c_void_p(0x10004), FAKE, None) == CP_ERR_ALIGN
    assert lib.cp_probe_copy(0, FAKE, FAKE, None) == CP_ERR_SHAPE


@needs_lib
def test_noalloc_ring_rejects_rows_beyond_its_scratch():
    """heads_q * chunk_len above CP_NOALLOC_MAX_ROWS is refused before any pointer is read."""
    lib = cp.load()
    r = cp.RingDesc(heads_q=1024, heads_kv=1024, chunk_len=(1 << 22) // 1024 + 1, head_dim=128,
                    n_cp=2, rank=1, causal=1, scale=0.0, dtype=cp.CP_BF16)
    st = lib.cp_attn_ring_bwd_noalloc(ctypes.byref(r), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, FAKE, None)
    assert st == -7 and "scratch" in cp.status_string(st)
    assert lib.cp_attn_ring_bwd_noalloc(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, None) == CP_ERR_NULL
