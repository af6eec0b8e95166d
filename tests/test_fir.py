"""Context-parallel causal FIR convolution (StripedHyena 2 context-parallelism page, section 3,
p2p convolution: only the first l_h - 1 outputs of a shard need the previous shard's tail).

CPU: pins of the fp64 oracle against things other than itself -- numpy's and scipy's own
convolution routines, the impulse response, the step response in closed form, causality, and a
brute-force scalar loop -- plus a check that the pins catch planted slips (a reversed filter, a
one-sample delay, a dropped tap) and that a shard without its halo differs from the oracle.
GPU (marked gpu): the local + halo kernels through the C ABI against the oracle.
"""
import numpy as np
import pytest
import scipy.signal

import oracle
from long_context_sequence_amd import inputs

RNG = np.random.default_rng(4321)


# ---- pins, written against an oracle callable so that the planted-slip test can reuse them

def pin_library(fir):
    for length, taps in ((37, 5), (16, 16), (9, 13), (64, 1)):
        x = RNG.standard_normal((3, length))
        h = RNG.standard_normal((3, taps))
        y = fir(x, h)
        for c in range(3):
            ref = np.convolve(x[c], h[c])[:length]
            if not np.allclose(y[c], ref, rtol=0, atol=1e-12):
                return False
            if not np.allclose(y[c], scipy.signal.lfilter(h[c], [1.0], x[c]), rtol=0, atol=1e-12):
                return False
    return True


def pin_impulse(fir):
    length, taps, t0 = 40, 7, 11
    h = RNG.standard_normal((2, taps))
    x = np.zeros((2, length))
    x[:, t0] = 1.0
    y = fir(x, h)
    want = np.zeros((2, length))
    want[:, t0:t0 + taps] = h
    return np.array_equal(y, want)


def pin_step(fir):
    length, taps = 30, 6
    h = RNG.standard_normal((2, taps))
    y = fir(np.ones((2, length)), h)
    want = np.stack([[h[c, :min(t, taps - 1) + 1].sum() for t in range(length)] for c in range(2)])
    return np.allclose(y, want, rtol=0, atol=1e-12)


def pin_causal(fir):
    x = RNG.standard_normal((2, 50))
    h = RNG.standard_normal((2, 9))
    y0 = fir(x, h)
    x2 = x.copy()
    x2[:, 20:] += RNG.standard_normal((2, 30))
    y1 = fir(x2, h)
    return np.array_equal(y0[:, :20], y1[:, :20]) and not np.allclose(y0[:, 20:], y1[:, 20:])


def pin_brute_force(fir):
    x = RNG.standard_normal((2, 12))
    h = RNG.standard_normal((2, 4))
    y = fir(x, h)
    for c in range(2):
        for t in range(12):
            acc = 0.0
            for k in range(4):
                if t - k >= 0:
                    acc += h[c, k] * x[c, t - k]
            if abs(acc - y[c, t]) > 1e-12:
                return False
    return True


PINS = [pin_library, pin_impulse, pin_step, pin_causal, pin_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pins(pin):
    assert pin(oracle.fir_forward)


def test_planted_slips_are_caught():
    def reversed_filter(x, h):
        return oracle.fir_forward(x, h[:, ::-1])

    def delayed(x, h):
        y = oracle.fir_forward(x, h)
        return np.concatenate([np.zeros((y.shape[0], 1)), y[:, :-1]], axis=1)

    def dropped_tap(x, h):
        return oracle.fir_forward(x, h[:, :-1]) if h.shape[1] > 1 else oracle.fir_forward(x, h)

    for slip in (reversed_filter, delayed, dropped_tap):
        assert not all(pin(slip) for pin in PINS), slip.__name__


def test_shards_reassemble_and_need_only_the_halo():
    """Per-shard outputs of the concatenated signal equal the zero-history convolution of the
    shard plus boundary terms that read only the previous shard's last l_h - 1 samples
    (brute force), and a shard-local convolution without them (a missing halo) differs."""
    n_cp, d, lc, taps = 4, 3, 10, 5
    xs = RNG.standard_normal((n_cp, d, lc))
    h = RNG.standard_normal((d, taps))
    ys = oracle.fir_shards(xs, h)
    full = oracle.fir_forward(np.concatenate(list(xs), axis=1), h)
    assert np.allclose(np.concatenate(list(ys), axis=1), full, rtol=0, atol=1e-12)
    for r in range(n_cp):
        local = oracle.fir_forward(xs[r], h)
        halo = np.zeros((d, lc))
        if r > 0:
            tail = xs[r - 1][:, lc - (taps - 1):]          # the l_h - 1 samples sent over
            for i in range(taps - 1):
                for k in range(i + 1, taps):
                    halo[:, i] += h[:, k] * tail[:, taps - 1 + i - k]
        assert np.allclose(ys[r], local + halo, rtol=0, atol=1e-12)
        if r > 0:
            assert not np.allclose(ys[r], local)


def test_fir_inputs_are_seeded_and_shaped():
    x, h = inputs.fir_inputs(7, 3, 4, 16, 5, "bf16")
    x2, h2 = inputs.fir_inputs(7, 3, 4, 16, 5, "bf16")
    assert x.shape == (3, 4, 16) and h.shape == (4, 5) and x.dtype == np.uint16
    assert np.array_equal(x, x2) and np.array_equal(h, h2)
    assert not np.array_equal(x[0], x[1])
    xf, hf = inputs.fir_inputs(7, 3, 4, 16, 5, "f32")
    assert np.array_equal(inputs.bf16_rne_bits(xf), x)


# ---- GPU parity through the C ABI

def _check_close(got, ref, what, rel=1e-5):
    err = np.max(np.abs(got - ref)) if ref.size else 0.0
    scale = max(1.0, float(np.max(np.abs(ref)))) if ref.size else 1.0
    assert err <= rel * scale, f"{what}: max err {err:.3g} (scale {scale:.3g})"


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("lc,taps", [(2100, 7), (2100, 128), (1001, 9), (64, 1), (15, 16),
                                     (4099, 1024), (1003, 33), (4100, 256), (40, 17), (31, 32),
                                     (9000, 257)])
def test_fir_ring_matches_oracle(dtype, lc, taps):
    import torch
    from long_context_sequence_amd import binding as cp

    n_cp, d = 4, 6
    xs, h = inputs.fir_inputs(900 + taps, n_cp, d, lc, taps, dtype)
    ref = oracle.fir_shards(inputs.widen(xs), inputs.widen(h))
    x_t, h_t = inputs.to_torch(xs, "cuda"), inputs.to_torch(h, "cuda")
    y = torch.full((n_cp, d, lc), float("nan"), device="cuda")
    halo = torch.empty((n_cp, d, taps - 1), dtype=x_t.dtype, device="cuda") if taps > 1 else None
    cp.fir_ring(x_t, h_t, halo, y)
    torch.cuda.synchronize()
    _check_close(y.cpu().numpy(), ref, f"ring {dtype} lc={lc} taps={taps}")


@pytest.mark.gpu
def test_fir_stages_separately():
    """Stage one alone is the zero-history convolution; the packed halo is the previous shard's
    tail; stage two completes the shard."""
    import torch
    from long_context_sequence_amd import binding as cp

    d, lc, taps = 5, 3000, 33
    xs, h = inputs.fir_inputs(77, 2, d, lc, taps, "bf16")
    xw, hw = inputs.widen(xs), inputs.widen(h)
    x_t, h_t = inputs.to_torch(xs, "cuda"), inputs.to_torch(h, "cuda")
    y = torch.empty((d, lc), device="cuda")
    cp.fir_local(x_t[1], h_t, y)
    torch.cuda.synchronize()
    _check_close(y.cpu().numpy(), oracle.fir_forward(xw[1], hw), "local stage")
    halo = torch.empty((d, taps - 1), dtype=torch.bfloat16, device="cuda")
    cp.fir_pack_halo(x_t[0], taps, halo)
    torch.cuda.synchronize()
    assert np.array_equal(halo.cpu().view(torch.int16).numpy().view(np.uint16), xs[0][:, lc - taps + 1:])
    cp.fir_halo(halo, h_t, y)
    torch.cuda.synchronize()
    _check_close(y.cpu().numpy(), oracle.fir_shards(xw, hw)[1], "local + halo")


@pytest.mark.gpu
@pytest.mark.parametrize("key", [12, 13])
def test_fir_full_size_share_sampled_channels(key):
    """The 208K-token share of rank 15 (D = 4096, 13,312 samples) in the benchmark's launch
    configuration (local stage over the whole share, halo from shard 14), checked on sampled
    channels against the oracle on shards 14 and 15 (enough history for l_h <= 13,313)."""
    import torch
    from long_context_sequence_amd import binding as cp
    from long_context_sequence_amd.configs import FIR_WORKLOADS

    wl = FIR_WORKLOADS[key]
    lc, d, taps = wl.shard_len, wl.channels, wl.taps
    r = wl.rank
    xs = {i: inputs.fir_shard(wl.key, i, d, lc, wl.dtype) for i in (r - 1, r)}
    h = inputs.fir_filters(wl.key, d, taps, wl.dtype)
    x_t, h_t = inputs.to_torch(xs[r], "cuda"), inputs.to_torch(h, "cuda")
    prev = inputs.to_torch(xs[r - 1], "cuda")
    y = torch.empty((d, lc), device="cuda")
    halo = torch.empty((d, taps - 1), dtype=torch.bfloat16, device="cuda")
    cp.fir_pack_halo(prev, taps, halo)
    cp.fir_local(x_t, h_t, y)
    cp.fir_halo(halo, h_t, y)
    torch.cuda.synchronize()
    chans = np.array([0, 1, d - 1] + list(np.random.default_rng(key).integers(0, d, 5)))
    pair = np.concatenate([inputs.widen(xs[r - 1][chans]), inputs.widen(xs[r][chans])], axis=1)
    ref = oracle.fir_forward(pair, inputs.widen(h[chans]))[:, lc:]
    _check_close(y[chans].cpu().numpy(), ref, wl.name)
