"""Plain fp64 CPU oracle for the context-parallel causal FIR convolution.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import this module. The GPU library never calls it and shares no code with it.

What the context-parallel convolution computes (StripedHyena 2 context-parallelism page,
section 3, the p2p convolution bullet): every channel of the sequence [D, L] is convolved
causally with its own finite impulse response h[c, 0 .. l_h - 1]. Cut along the sequence into
N_cp shards, the convolution of a shard is local except for its first l_h - 1 outputs, which
also need the last l_h - 1 inputs of the previous shard. That split is how the GPU path computes
(a zero-padded local convolution, then the boundary terms once the neighbour's tail arrives);
the oracle is the plain definition over the whole concatenated sequence:

    y[c, t] = sum_{k = 0}^{l_h - 1} h[c, k] * x[c, t - k],   with x[c, t'] = 0 for t' < 0.

Reading of what the page leaves open: the filter taps multiply the current and earlier inputs
(h[c, 0] weighs x[c, t]); the first shard has no predecessor (zero history).
"""
from __future__ import annotations

import numpy as np


def fir_forward(x, h) -> np.ndarray:
    """Causal depthwise convolution of x [D, L] with h [D, l_h]; returns y [D, L] in fp64."""
    x = np.asarray(x, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    if x.ndim != 2 or h.ndim != 2 or x.shape[0] != h.shape[0]:
        raise ValueError("x must be [D, L] and h [D, l_h] with the same D")
    n_ch, length = x.shape
    y = np.zeros((n_ch, length), dtype=np.float64)
    for k in range(min(h.shape[1], length)):
        # tap k: x delayed by k samples, zero before the start
        y[:, k:] += h[:, k:k + 1] * x[:, :length - k]
    return y


def fir_shards(x_shards, h) -> np.ndarray:
    """Per-shard outputs [N_cp, D, Lc] of the convolution of the concatenated shards
    x_shards [N_cp, D, Lc] (shard r holds positions r*Lc .. r*Lc + Lc - 1)."""
    x_shards = np.asarray(x_shards, dtype=np.float64)
    n_cp, n_ch, lc = x_shards.shape
    full = np.concatenate(list(x_shards), axis=1)           # [D, N_cp * Lc]
    y = fir_forward(full, h)
    return np.stack([y[:, r * lc:(r + 1) * lc] for r in range(n_cp)])
