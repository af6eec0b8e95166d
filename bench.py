"""Throughput of one context-parallel rank's ring attention on one MI355X.

A timed step is one pass of the rank's whole hot path over its synthetic inputs: the forward
ring (every visited chunk: the step kernel folding into the running (O, LSE)) and, when the
workload has one, the backward ring (delta prep, then the backward kernels per visited chunk,
into zeroed fp32 dQ/dK/dV). Inputs are resident in HBM before the timed region starts.

Default workload: rank 15 of a 212,992-token sequence in 16 chunks of 13,312 (32 query heads,
8 key/value heads, d = 128, causal), forward + backward.

Prints one JSON line. `value` is fwd+bwd algorithmic TFLOP/s (visible query-key pairs only:
4*d*H_q flops per pair forward, 10*d*H_q backward); the forward and backward rates, tokens/s and
the per-kernel roofline ride along. HIP events recorded on the launch stream around every step
kernel inside the timed region give the per-kernel durations.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
PEAK_F32_VALU_TFLOPS = 157.3  # MI355X fp32 vector (published; counts packed FMA)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=4, help="named workload key (2..5)")
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--fwd-only", action="store_true")
    ap.add_argument("--separate-merge", action="store_true",
                    help="step into scratch + cp_attn_merge instead of the fused fold")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the oracle CPU baseline (0 disables it)")
    ap.add_argument("--no-merge-bench", action="store_true")
    ap.add_argument("--no-fir-bench", action="store_true",
                    help="skip the causal FIR convolution leg (short and medium filters)")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the sustained-rate probes (MFMA-only kernel, 1 GiB copy)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy first (reference for HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs one rank's ring on one GPU; "
                                   "multi-GPU runs are not supported (use --gpus 1)"}))
        sys.exit(2)
    import torch

    from long_context_sequence_amd import binding as cp
    from long_context_sequence_amd import configs, inputs

    wl = configs.WORKLOADS[args.workload]
    rank = wl.ranks[-1] if args.rank is None else args.rank
    do_bwd = not args.fwd_only
    n_workers = host_workers()
    pool = start_oracle_pool(n_workers) if args.cpu_seconds > 0 else None
    dev = "cuda"
    torch.cuda.set_device(0)
    cp.load()

    t0 = time.time()
    q = inputs.to_torch(inputs.workload_tensor(wl, "q", rank), dev)
    kc = inputs.to_torch(inputs.workload_kv(wl, "k"), dev)
    vc = inputs.to_torch(inputs.workload_kv(wl, "v"), dev)
    d_o = inputs.to_torch(inputs.workload_tensor(wl, "do", rank), dev)
    print(f"# inputs ready in {time.time() - t0:.1f}s: q {tuple(q.shape)} kv {tuple(kc.shape)}",
          file=sys.stderr, flush=True)
    hq, lc, d = q.shape
    o = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    o_work = torch.empty_like(o) if args.separate_merge else None
    lse_work = torch.empty_like(lse) if args.separate_merge else None
    delta = torch.empty_like(lse)
    dq = torch.zeros_like(o)
    dk = torch.zeros(kc.shape, dtype=torch.float32, device=dev)
    dv = torch.zeros(kc.shape, dtype=torch.float32, device=dev)

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        a.fill_(1.0)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    sched = [(c, cls) for c, cls in cp.ring_schedule(wl.n_cp, rank, wl.causal)
             if cls != configs.SKIP]

    def step_flops(c):
        # visible pairs per head of this chunk for this rank
        if not wl.causal or c < rank:
            return lc * lc
        return lc * (lc + 1) // 2

    fwd_step_flops = [4.0 * d * hq * step_flops(c) for c, _ in sched]
    bwd_step_flops = [10.0 * d * hq * step_flops(c) for c, _ in sched]

    # probe once whether the backward kernels exist in this build
    if do_bwd:
        try:
            cp.bwd(q, kc[rank], vc[rank], d_o, lse, delta, dq, dk[rank], dv[rank],
                   q_pos0=rank * lc, kv_pos0=rank * lc, causal=wl.causal)
        except cp.CpAttnError as e:
            if e.status != -5:
                raise
            do_bwd = False
            print("# backward kernels not in this build: timing the forward only",
                  file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    def run_step(ev_f=None, ev_b=None):
        first = True
        for i, (c, _) in enumerate(sched):
            if ev_f is not None:
                ev_f[i][0].record(stream)
            if first or not args.separate_merge:
                cp.step(q, kc[c], vc[c], o, lse, q_pos0=rank * lc, kv_pos0=c * lc,
                        causal=wl.causal, accumulate=not first)
            else:
                cp.step(q, kc[c], vc[c], o_work, lse_work, q_pos0=rank * lc, kv_pos0=c * lc,
                        causal=wl.causal)
            if ev_f is not None:
                ev_f[i][1].record(stream)
            if not first and args.separate_merge:
                cp.merge(o, lse, o_work, lse_work)
            first = False
        if do_bwd:
            dq.zero_()
            dk.zero_()
            dv.zero_()
            cp.bwd_prep(o, d_o, delta)
            for i, (c, _) in enumerate(sched):
                if ev_b is not None:
                    ev_b[i][0].record(stream)
                cp.bwd(q, kc[c], vc[c], d_o, lse, delta, dq, dk[c], dv[c], q_pos0=rank * lc,
                       kv_pos0=c * lc, causal=wl.causal)
                if ev_b is not None:
                    ev_b[i][1].record(stream)

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    evs_f = [[(mk(), mk()) for _ in sched] for _ in range(args.steps)]
    evs_b = [[(mk(), mk()) for _ in sched] for _ in range(args.steps)]
    start, end = mk(), mk()
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(args.steps):
        run_step(evs_f[s], evs_b[s] if do_bwd else None)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    fwd_ms = sum(a.elapsed_time(b) for st in evs_f for a, b in st) / args.steps
    bwd_ms = (sum(a.elapsed_time(b) for st in evs_b for a, b in st) / args.steps) if do_bwd else 0.0
    f_fwd = sum(fwd_step_flops)
    f_bwd = sum(bwd_step_flops) if do_bwd else 0.0
    print(f"# timed {args.steps} steps: {ms_step:.2f} ms/step (fwd kernels {fwd_ms:.2f} ms, "
          f"bwd kernels {bwd_ms:.2f} ms)", file=sys.stderr, flush=True)

    # Dominant kernel: the one with the largest share of the step. Algorithmic flops per launch:
    # forward 4*d*H_q per visible pair (QK^T, PV); backward 10*d*H_q (S recompute, dP, dV, dK,
    # dQ), one bwd_kernel launch per ring step. Summed over the step's launches / summed
    # durations.
    cands = [("fwd_bf16_kernel (cp_attn_step)", fwd_ms, f_fwd)]
    if do_bwd:
        cands.append(("bwd_kernel (cp_attn_bwd)", bwd_ms, f_bwd))
    dom_name, dom_ms, dom_flops = max(cands, key=lambda c: c[1])
    n_launch = len(sched)
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    traffic = measured_traffic(wl.name, dom_name.split(" ")[0])
    roofline = {"bound": "mfma", "kernel": dom_name, "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic["total_bytes"] if traffic else None,
                "traffic_read_write": ([traffic["read_bytes"], traffic["write_bytes"]]
                                       if traffic else None),
                "launches_per_step": n_launch,
                "avg_launch_ms": round(dom_ms / n_launch, 4)}

    merge_info = None
    if not args.no_merge_bench:
        merge_info = bench_merge(cp, torch, o, lse, wl.name)

    fir_info = None
    if not args.no_fir_bench:
        fir_info = [bench_fir(cp, torch, configs.FIR_WORKLOADS[k]) for k in (12, 13)]

    probe = None
    if not args.no_probe:
        probe = device_probe(cp, torch)
        roofline["sustained_peak"] = probe["mfma_bf16_TFLOPs"]
        roofline["frac_of_sustained"] = round(achieved / probe["mfma_bf16_TFLOPs"], 4)

    cpu = None
    if pool is not None:
        cpu = cpu_baseline(pool, n_workers, wl, rank, args.cpu_seconds, do_bwd)
        pool.close()
        pool.join()

    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    out = {
        "metric": "ring-step causal attention TFLOP/s (fwd+bwd) per rank",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 Q/K/V/dO",
        "config": {"workload": wl.name, "seq_len": wl.seq_len, "n_cp": wl.n_cp, "rank": rank,
                   "chunk_len": lc, "heads_q": hq, "heads_kv": wl.heads_kv, "head_dim": d,
                   "causal": wl.causal, "backward": do_bwd,
                   "merge": "separate" if args.separate_merge else "fused"},
        "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2),
        "fwd_frac_of_peak": round(f_fwd / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "bwd_tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2) if do_bwd else None,
        "kernel_ms_per_step": {"fwd": round(fwd_ms, 3), "bwd": round(bwd_ms, 3)},
        "bwd_frac_of_peak": (round(f_bwd / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
                             if do_bwd else None),
        "tokens_per_s": round(lc / (ms_step * 1e-3), 1),
        "roofline": roofline,
        "merge_kernel": merge_info,
        "fir_conv": fir_info,
        "device_probe": probe,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


KERNEL_SOURCES = {"fwd_bf16_kernel": "fwd_bf16.hip", "bwd_kernel": "bwd_bf16.hip",
                  "merge_kernel": "elementwise.hip", "prep_kernel": "elementwise.hip",
                  "fir_local_kernel": "fir.hip", "fir_local_mfma_kernel": "fir.hip",
                  "fir_pack_kernel": "fir.hip", "fir_halo_kernel": "fir.hip"}


def measured_traffic(workload_name, kernel):
    """HBM bytes per launch (read + written) of `kernel` from the committed rocprofv3 counter
    summary of this workload (FETCH_SIZE / WRITE_SIZE scaled by a 1 GiB copy), or None when no
    summary exists or the kernel's source changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"{workload_name}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("kernels", {}).get(kernel)
    if rec is None or kernel not in KERNEL_SOURCES:
        return None
    h = hashlib.sha1()
    csrc = os.path.join(ROOT, "long_context_sequence_amd", "csrc")
    for name in (KERNEL_SOURCES[kernel], "device_common.hpp", "kernels.hpp"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["source_sha1"]:
        return None
    return {"read_bytes": int(rec["read_bytes"]), "write_bytes": int(rec["write_bytes"]),
            "total_bytes": int(rec["read_bytes"] + rec["write_bytes"])}


def bench_fir(cp, torch, wl, reps=20):
    """One rank's share of the causal FIR convolution (rank 15 of 16: D channels x 13,312
    samples): pack the tail for the next rank, the local stage, the halo stage with the previous
    shard's tail. HIP events on the launch stream around each kernel. Algorithmic bytes: x read
    and y written once (plus the halo); flops 2 * taps per output."""
    from long_context_sequence_amd import inputs

    r, d, lc, taps = wl.rank, wl.channels, wl.shard_len, wl.taps
    x = inputs.to_torch(inputs.fir_shard(wl.key, r, d, lc, wl.dtype), "cuda")
    prev = inputs.to_torch(inputs.fir_shard(wl.key, r - 1, d, lc, wl.dtype), "cuda")
    h = inputs.to_torch(inputs.fir_filters(wl.key, d, taps, wl.dtype), "cuda")
    y = torch.empty((d, lc), device="cuda")
    halo_in = torch.empty((d, taps - 1), dtype=x.dtype, device="cuda")
    halo_out = torch.empty_like(halo_in)
    stream = torch.cuda.current_stream()
    cp.fir_pack_halo(prev, taps, halo_in)          # what rank r - 1 would have sent
    for _ in range(3):
        cp.fir_pack_halo(x, taps, halo_out)
        cp.fir_local(x, h, y)
        cp.fir_halo(halo_in, h, y)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record(stream)
        cp.fir_pack_halo(x, taps, halo_out)
        ev[i][1].record(stream)
        cp.fir_local(x, h, y)
        ev[i][2].record(stream)
        cp.fir_halo(halo_in, h, y)
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    pack = sum(e[0].elapsed_time(e[1]) for e in ev) / reps
    local = sum(e[1].elapsed_time(e[2]) for e in ev) / reps
    halo = sum(e[2].elapsed_time(e[3]) for e in ev) / reps
    share = pack + local + halo
    elem = 2 if wl.dtype == "bf16" else 4
    local_bytes = d * lc * (elem + 4)
    local_flops = 2.0 * taps * d * lc
    gbs = local_bytes / (local * 1e-3) / 1e9
    tfl = local_flops / (local * 1e-3) / 1e12
    # the local stage runs on the matrix cores for bf16 filters of 17..256 taps (Toeplitz
    # product), on the fp32 VALU otherwise; its compute roof is the matching peak
    on_mfma = wl.dtype == "bf16" and 16 < taps <= 256
    unit, peak = ("mfma", PEAK_BF16_TFLOPS) if on_mfma else ("alu", PEAK_F32_VALU_TFLOPS)
    hbm_frac, alu_frac = gbs / PEAK_HBM_GBS, tfl / peak
    bound = "hbm" if hbm_frac >= alu_frac else unit
    return {"workload": wl.name, "channels": d, "shard_len": lc, "taps": taps,
            "ms_pack": round(pack, 4), "ms_local": round(local, 4), "ms_halo": round(halo, 4),
            "ms_share": round(share, 4),
            "local_kernel": {"bound": bound, "units": unit, "achieved_GBs": round(gbs, 1),
                             "hbm_frac": round(hbm_frac, 4), "achieved_TFLOPs": round(tfl, 2),
                             "compute_frac": round(alu_frac, 4),
                             "bytes_per_launch": local_bytes},
            "samples_per_s": round(d * lc / (share * 1e-3), 1)}


def device_probe(cp, torch, reps=3):
    """What this device sustains, beside the published peaks that the roofline fractions use:
    a kernel of nothing but register-fed 32x32x16 bf16 MFMAs on every CU (cp_probe_mfma_bf16),
    and a 1 GiB copy with 16-byte accesses (cp_probe_copy; 2 GiB moved per copy)."""
    stream = torch.cuda.current_stream()
    n_wg, iters = 256 * 8, 2048
    sink = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    cp.probe_mfma_bf16(n_wg, 64, sink)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    flops = sum(cp.probe_mfma_bf16(n_wg, iters, sink) for _ in range(reps))
    t1.record(stream)
    t1.synchronize()
    mfma_tf = flops / (t0.elapsed_time(t1) * 1e-3) / 1e12
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    cp.probe_copy(a, b)
    torch.cuda.synchronize()
    t0.record(stream)
    moved = sum(cp.probe_copy(a, b) for _ in range(reps))
    t1.record(stream)
    t1.synchronize()
    copy_gbs = moved / (t0.elapsed_time(t1) * 1e-3) / 1e9
    del a, b, sink
    return {"mfma_bf16_TFLOPs": round(mfma_tf, 1), "mfma_frac_of_published": round(mfma_tf / PEAK_BF16_TFLOPS, 4),
            "copy_GBs": round(copy_gbs, 1), "copy_frac_of_published": round(copy_gbs / PEAK_HBM_GBS, 4)}


def bench_merge(cp, torch, o, lse, workload_name):
    """cp_attn_merge alone on the rank's (O, LSE) shapes: GB/s of algorithmic traffic
    (read O_acc, O_step, both LSEs; write O_acc, LSE_acc: 12 B per O element + 12 B per row),
    beside the HBM bytes per launch that rocprofv3's FETCH_SIZE/WRITE_SIZE counters measured
    for this kernel on the same shapes (committed summary; None once the source changed)."""
    o2 = torch.randn_like(o)
    l2 = torch.randn_like(lse)
    oa = torch.randn_like(o)
    la = torch.randn_like(lse)
    for _ in range(2):
        cp.merge(oa, la, o2, l2)
    torch.cuda.synchronize()
    n = 10
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(n):
        cp.merge(oa, la, o2, l2)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / n
    byts = 12.0 * o.numel() + 12.0 * lse.numel()
    gbs = byts / (ms * 1e-3) / 1e9
    traffic = measured_traffic(workload_name, "merge_kernel")
    return {"bound": "hbm", "avg_launch_ms": round(ms, 4), "bytes_per_launch": int(byts),
            "achieved_GBs": round(gbs, 1), "peak_GBs": PEAK_HBM_GBS,
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic["total_bytes"] if traffic else None,
            "traffic_read_write": ([traffic["read_bytes"], traffic["write_bytes"]]
                                   if traffic else None)}


def host_workers() -> int:
    """Host cores of this process's share (at most 16: one GPU's share of a host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def start_oracle_pool(n):
    """n worker processes for the oracle baseline, started before anything touches the GPU (so
    they inherit no GPU state); each holds BLAS to one thread."""
    import multiprocessing

    return multiprocessing.get_context("spawn").Pool(n, initializer=_oracle_worker_init)


def _oracle_worker_init():
    from threadpoolctl import threadpool_limits

    global _BLAS_LIMIT
    _BLAS_LIMIT = threadpool_limits(limits=1, user_api="blas")


_ORACLE_KV = {}


def _oracle_block(task):
    """One sampled block: `rows` consecutive query rows of query head h of the rank, forward and
    (with_bwd) backward of the fp64 oracle against every key of the sequence. Returns (visible
    pairs, seconds)."""
    import oracle
    from long_context_sequence_amd import configs, inputs

    key, rank, h, i0, rows, with_bwd = task
    wl = configs.WORKLOADS[key]
    g = h // wl.group
    if (key, g) not in _ORACLE_KV:
        _ORACLE_KV.clear()
        kf = np.concatenate([inputs.widen(inputs.workload_tensor(wl, "k", c)[g:g + 1])
                             for c in range(wl.n_cp)], axis=1)
        vf = np.concatenate([inputs.widen(inputs.workload_tensor(wl, "v", c)[g:g + 1])
                             for c in range(wl.n_cp)], axis=1)
        _ORACLE_KV[(key, g)] = (kf, vf)
    kf, vf = _ORACLE_KV[(key, g)]
    lc = wl.chunk_len
    qb = inputs.widen(inputs.workload_tensor(wl, "q", rank)[h:h + 1, i0:i0 + rows])
    db = inputs.widen(inputs.workload_tensor(wl, "do", rank)[h:h + 1, i0:i0 + rows])
    q0 = rank * lc + i0
    nkeys = kf.shape[1]
    pairs = sum(min(nkeys, q0 + i + 1) if wl.causal else nkeys for i in range(qb.shape[1]))
    t = time.perf_counter()
    oracle.attention_forward(qb, kf, vf, q_pos0=q0, causal=wl.causal, scale=wl.scale)
    if with_bwd:
        oracle.attention_backward(qb, kf, vf, db, q_pos0=q0, causal=wl.causal, scale=wl.scale)
    return pairs, time.perf_counter() - t


def cpu_baseline(pool, n_workers, wl, rank, budget_s, with_bwd):
    """The fp64 oracle on the host cores, on a bounded, seeded sample of the same workload: one
    block of consecutive query rows per worker process (one BLAS thread each), every row against
    all its visible keys, forward and backward. The rate is the sample's algorithmic flops (the
    GPU metric's count: 4*d forward + 10*d backward per visible pair) over the wall time of the
    whole pool; the rank's full work at that rate is reported as an extrapolation."""
    d, lc = wl.head_dim, wl.chunk_len
    # block height: about budget_s of work per worker at ~12 GFLOP/s per core (fp64 numpy)
    per_pair = (14.0 if with_bwd else 4.0) * d
    visible = rank * lc + lc // 2 if wl.causal else wl.seq_len
    rows = int(max(16, min(lc, budget_s * 12e9 / (per_pair * visible))))
    rng = np.random.default_rng(0)
    # heads of one key/value group, so that every worker needs the same K and V (generated once
    # per worker by the warm-up map, outside the timed region)
    g = int(rng.integers(0, wl.heads_kv))
    tasks = [(wl.key, rank, g * wl.group + i % wl.group, int(rng.integers(0, lc - rows + 1)),
              rows, with_bwd) for i in range(n_workers)]
    pool.map(_oracle_block, [(wl.key, rank, t[2], 0, 1, False) for t in tasks], chunksize=1)
    t0 = time.perf_counter()
    res = pool.map(_oracle_block, tasks, chunksize=1)
    wall = time.perf_counter() - t0
    flops = per_pair * sum(pr for pr, _ in res)
    rate = flops / wall
    rank_pairs = (rank * lc * lc + lc * (lc + 1) // 2) if wl.causal else wl.n_cp * lc * lc
    full = per_pair * wl.heads_q * rank_pairs / rate
    return {"value": round(rate / 1e12, 5), "unit": "TFLOP/s", "cores": n_workers,
            "kind": "oracle", "workers": n_workers, "blas_threads_per_worker": 1,
            "wall_s": round(wall, 2), "gflops_fp64": round(rate / 1e9, 1),
            "extrapolated_full_rank_s": round(full, 1),
            "sample": f"{n_workers} blocks of {rows} query rows (one per worker process) x all "
                      f"visible keys, {'fwd+bwd' if with_bwd else 'fwd'}, fp64 numpy; the full "
                      f"rank's time is extrapolated from this rate"}


if __name__ == "__main__":
    main()
