"""Seeded input generators and workload arithmetic (CPU only)."""
import numpy as np
import torch

from long_context_sequence_amd import configs, inputs


def test_bf16_rounding_ties_to_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)
    x = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + 2.0 ** -20,
                  -(one + ulp / 2), 3.140625, 1e-30], dtype=np.float32)
    got = inputs.bf16_bits_to_f32(inputs.bf16_rne_bits(x))
    want = np.array([1.0, 1.0, 1.0 + 2 * 2.0 ** -7, 1.0 + 2.0 ** -7, -1.0, 3.140625,
                     np.float32(1e-30)], dtype=np.float32)
    assert np.array_equal(got[:6], want[:6])
    # matches torch's float32 -> bfloat16 conversion on random data
    r = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    tb = torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(inputs.bf16_rne_bits(r), tb)


def test_generation_is_deterministic_and_distinct():
    a = inputs.make(3, "k", 2, (2, 5, 8), "bf16")
    b = inputs.make(3, "k", 2, (2, 5, 8), "bf16")
    c = inputs.make(3, "k", 3, (2, 5, 8), "bf16")
    d = inputs.make(3, "v", 2, (2, 5, 8), "bf16")
    assert np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)


def test_rms_rows():
    x = inputs.rms_rows(inputs.normal_f32(9, "q", 0, (3, 50, 128)))
    ms = np.mean(x.astype(np.float64) ** 2, axis=-1)
    assert np.allclose(ms, 1.0, atol=1e-4)


def test_workload_shapes_and_flops():
    c4 = configs.C4
    assert c4.chunk_len == 13312 and c4.group == 4
    assert inputs.shard_shape(c4, "q") == (32, 13312, 128)
    assert inputs.shard_shape(c4, "k") == (8, 13312, 128)
    # 45.00 TFLOP forward for rank 15 of the 208K sequence
    assert abs(configs.fwd_flops(c4, 15) / 1e12 - 45.00) < 0.01
    assert abs(configs.fwd_flops(configs.C3, 7) / 1e12 - 2.062) < 0.001
    assert configs.visible_pairs(configs.C1, 0) == 64 * 256


def test_ring_schedule_reading():
    # rank 0 of 4, non-causal: chunks 0, 3, 2, 1, all fully visible
    assert configs.ring_schedule(4, 0, False) == [(0, 0), (3, 0), (2, 0), (1, 0)]
    sched = configs.ring_schedule(16, 15, True)
    assert sched[0] == (15, configs.DIAG)
    assert all(cls == configs.FULL for _, cls in sched[1:])
    for n in (1, 3, 8):
        for r in range(n):
            s = configs.ring_schedule(n, r, True)
            assert sorted(c for c, _ in s) == list(range(n))
            assert [c for c, cls in s if cls != configs.SKIP] == list(range(r, -1, -1))
