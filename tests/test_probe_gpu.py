"""The rate probes run through the C ABI and do the work they claim. Matrix cores: every
iteration adds the same A*B into each accumulator, so two iterations give exactly twice the
per-thread sums of one (doubling is exact in fp32). Copy: the destination equals the source,
including a ragged last workgroup."""
import pytest
import torch

from long_context_sequence_amd import binding as cp

pytestmark = pytest.mark.gpu


def test_probe_mfma_linear_in_iterations():
    n_wg = 8
    s1 = torch.full((n_wg * 256,), float("nan"), dtype=torch.float32, device="cuda")
    s2 = torch.full_like(s1, float("nan"))
    f1 = cp.probe_mfma_bf16(n_wg, 1, s1)
    f2 = cp.probe_mfma_bf16(n_wg, 2, s2)
    torch.cuda.synchronize()
    assert f2 == 2 * f1 == 2.0 * n_wg * 4 * 4 * 32768
    assert torch.isfinite(s1).all() and (s1 != 0).any()
    assert torch.equal(s2, 2 * s1)


def test_probe_copy_exact():
    src = torch.randn(4 * 1000, dtype=torch.float32, device="cuda")
    dst = torch.zeros_like(src)
    assert cp.probe_copy(src, dst) == 32.0 * 1000
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
