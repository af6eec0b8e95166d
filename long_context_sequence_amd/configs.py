"""The five ring-attention workloads and the ring schedule's host arithmetic.

A workload is one context-parallel (CP) job: a sequence of ``seq_len`` tokens cut into ``n_cp``
contiguous chunks of ``chunk_len`` tokens (StripedHyena 2 context-parallelism page, section 1:
the input [D, L] is split along the sequence into N_cp shards of [D, L/N_cp]). A rank keeps its
query shard and, one ring step at a time, attends to the key/value chunk it currently holds
(same page, section 2, "ring attention" steps 1-4).

Nothing here computes attention; it only names sizes and counts work for the throughput report.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    key: int                 # seed namespace of the inputs (1..5 for the named workloads)
    name: str
    dtype: str               # "f32" or "bf16": the type Q, K, V (and dO) are stored in
    heads_q: int
    heads_kv: int
    head_dim: int
    seq_len: int
    n_cp: int
    causal: bool
    ranks: tuple             # ranks whose share is run
    rms_rows: bool = False   # per-token RMS-normalised Q/K/V rows
    backward: bool = False
    note: str = field(default="", compare=False)

    @property
    def chunk_len(self) -> int:
        return self.seq_len // self.n_cp

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    @property
    def scale(self) -> float:
        return 1.0 / (self.head_dim ** 0.5)


C1 = Workload(1, "tiny-noncausal-f32", "f32", 2, 2, 64, 256, 4, False, (0,),
              note="rank 0 of 4, fp32, non-causal, ring order 0,3,2,1")
C2 = Workload(2, "mha-causal-8k", "bf16", 32, 32, 128, 8192, 8, True, tuple(range(8)),
              note="all 8 ranks, MHA")
C3 = Workload(3, "gqa-causal-32k-rms", "bf16", 32, 8, 128, 32768, 8, True, (7,), rms_rows=True,
              note="last rank, GQA group 4, RMS-normalised rows")
C4 = Workload(4, "gqa-causal-208k-rank15", "bf16", 32, 8, 128, 212992, 16, True, (15,),
              note="rank 15 of 16: 13,312 queries against 212,992 keys")
C5 = Workload(5, "gqa-causal-32k-fwd-bwd", "bf16", 32, 8, 128, 32768, 8, True, (7,), backward=True,
              note="last rank, forward + backward")

WORKLOADS = {w.key: w for w in (C1, C2, C3, C4, C5)}

# The ring schedule's step classes.
FULL, DIAG, SKIP = 0, 1, 2


def ring_schedule(n_cp: int, rank: int, causal: bool):
    """Chunk held at each ring step and its causal class.

    A rank receives from its predecessor, so at step s it holds chunk (rank - s) mod n_cp
    (ring attention, step 1 on the context-parallelism page). Under causal masking with
    contiguous chunks a chunk after the rank's own is entirely in the future (SKIP), the rank's
    own chunk needs the triangular mask (DIAG), earlier ones are fully visible (FULL).
    """
    out = []
    for s in range(n_cp):
        c = (rank - s) % n_cp
        if not causal or c < rank:
            cls = FULL
        elif c == rank:
            cls = DIAG
        else:
            cls = SKIP
        out.append((c, cls))
    return out


def visible_pairs(wl: Workload, rank: int) -> int:
    """(query, key) pairs per head that the rank's queries may attend to."""
    lc = wl.chunk_len
    if not wl.causal:
        return lc * wl.seq_len
    return rank * lc * lc + lc * (lc + 1) // 2


def fwd_flops(wl: Workload, rank: int) -> float:
    """Algorithmic forward flops: QK^T and PV, 2*d each per visible pair and query head."""
    return 4.0 * wl.head_dim * wl.heads_q * visible_pairs(wl, rank)


def bwd_flops(wl: Workload, rank: int) -> float:
    """Algorithmic backward flops: the S recompute, dP, dV, dK and dQ products (2*d each)."""
    return 10.0 * wl.head_dim * wl.heads_q * visible_pairs(wl, rank)


# ---- causal FIR convolution workloads (StripedHyena 2 context-parallelism page, section 3:
# the p2p convolution of the short explicit and medium regularized filters). The page names the
# filter classes but not their lengths; "short" is taken as 7 taps and "medium" as 128.

@dataclass(frozen=True)
class FirWorkload:
    key: int
    name: str
    dtype: str          # of x, h and the halo
    channels: int       # D
    seq_len: int
    n_cp: int
    taps: int           # l_h
    rank: int           # the rank whose share is benchmarked
    note: str = field(default="", compare=False)

    @property
    def shard_len(self) -> int:
        return self.seq_len // self.n_cp

    def flops(self) -> float:
        """Algorithmic flops of one rank's share: 2 * taps per output (the causal ramp at the
        start of the sequence is ignored)."""
        return 2.0 * self.taps * self.channels * self.shard_len

    def bytes(self) -> float:
        """Algorithmic HBM bytes of one rank's share: x read once, y written once (fp32), the
        halo read (plus the tail packed for the next rank)."""
        e = 2 if self.dtype == "bf16" else 4
        return self.channels * (self.shard_len * (e + 4) + 2 * (self.taps - 1) * e)


F1 = FirWorkload(11, "fir-tiny-f32", "f32", 4, 256, 4, 5, 3, note="fp32, 4 shards of 64")
F2 = FirWorkload(12, "fir-short-208k", "bf16", 4096, 212992, 16, 7, 15,
                 note="D = 4096, 16 shards of 13,312, 7 taps")
F3 = FirWorkload(13, "fir-medium-208k", "bf16", 4096, 212992, 16, 128, 15,
                 note="D = 4096, 16 shards of 13,312, 128 taps")
FIR_WORKLOADS = {w.key: w for w in (F1, F2, F3)}
