#!/usr/bin/env python3
"""Benchmark: achieved KV-cache HBM bandwidth and time per split-K paged decode step on one
MI355X, with the roofline of the dominant kernel and the float64 CPU oracle beside it.

A step is one pass of the decode hot path over one batch: paged_decode_partial followed by
paged_decode_reduce on the same stream. The headline workload is the Llama-style GQA batch
(B=32, H=32, KVH=8, D=128, bf16, lengths U[512, 4096], partition 512). The batch's KV pool
is kept in R copies at different HBM addresses and the steps cycle through them (as
successive layers of a model would), so that the 256 MB Infinity Cache cannot serve one
step's KV from the previous step; every copy is resident before timing starts.

Prints exactly one JSON line (rank 0, N = 1). ``--gpus N`` with N > 1 exits with a message:
this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, AMD published
MALL_BYTES = 256 * 2**20


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama_gqa4",
                    choices=["llama_gqa4", "wide_gqa6", "skewed_gqa8", "tiny_fp32", "mla_prefill_b8", "mla_decode_b64"])
    ap.add_argument("--copies", type=int, default=0, help="KV pool copies to cycle (0 = auto)")
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--eager", action="store_true", help="time eager submission instead of a HIP graph replay")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time to spend")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy of MIB MiB (read MIB, write MIB) a few times, "
                         "to scale HBM byte counters read under a profiler")
    return ap.parse_args()


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def bench_decode(case, steps, warmup, copies=0, one_launch=False, graph=True):
    """Time `steps` decode steps; returns a dict of measurements. A step is the two phases
    (paged_decode_partial + paged_decode_reduce), or with `one_launch` the single-launch
    paged_decode (phase 1 with the combine done by the last workgroup of each (sequence,
    kv head)); the timed kernel is then that one launch.

    With `graph`, the `steps` steps are captured once into a HIP graph and the timed region
    is one replay of it (a decode loop submits its kernels that way; eager submission from
    Python adds tens of microseconds of host latency before the first kernel, which at 20
    steps is over a microsecond per step). The graph is replayed once untimed first, and the
    output of the timed replay must equal, bit for bit, an eager run of its last step. The
    eager time of the same steps is reported beside it."""
    import torch
    import paged_kv_gqa_table_amd as pkv

    dev = "cuda"
    q = case.query.to(dev)
    bt = case.block_tables.to(dev)
    lens = case.seq_lens.to(dev)
    k0 = case.key_cache.to(dev)
    v0 = case.value_cache.to(dev)
    pool_bytes = 2 * k0.numel() * k0.element_size()
    if copies <= 0:
        copies = max(1, min(8, math.ceil(3 * MALL_BYTES / max(1, pool_bytes))))
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]
    S, H, D = case.num_seqs, case.num_heads, case.head_dim
    ps = case.partition_size
    max_len = case.max_seq_len
    P = case.num_partitions()
    acc = torch.empty((S, H, P, D), dtype=torch.float32, device=dev)
    m = torch.empty((S, H, P), dtype=torch.float32, device=dev)
    l = torch.empty((S, H, P), dtype=torch.float32, device=dev)
    out = torch.empty((S, H, D), dtype=case.query.dtype, device=dev)
    counters = torch.zeros((S * case.num_kv_heads,), dtype=torch.int32, device=dev)

    def step(i, ev=None):
        kc, vc = pools[i % copies]
        if ev is not None:
            ev[0].record()
        if one_launch:
            pkv.paged_decode_into(q, kc, vc, bt, lens, case.scale, case.num_kv_heads, ps, 0, max_len, out, None,
                                  acc, m, l, counters, layout=case.layout)
            if ev is not None:
                ev[1].record()
            return
        pkv.paged_decode_partial(q, kc, vc, bt, lens, case.scale, case.num_kv_heads, ps, max_len,
                                 acc, m, l, layout=case.layout)
        if ev is not None:
            ev[1].record()
        pkv.paged_decode_reduce(acc, m, l, lens, ps, out)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    def timed_eager():
        t_start, t_end = _events(2)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        t_start.record()
        for i in range(steps):
            step(i)
        t_end.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, t_start.elapsed_time(t_end)

    # Region 1 (the contract): exactly `steps` back-to-back steps between two synchronizes.
    eager_wall, eager_gpu_ms = timed_eager()
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                step(i)
        g.replay()  # untimed: the first replay uploads the graph
        torch.cuda.synchronize()
        t_start, t_end = _events(2)
        t0 = time.perf_counter()
        t_start.record()
        g.replay()
        t_end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu_ms = t_start.elapsed_time(t_end)
        got = out.clone()
        step(steps - 1)  # the graph's last step, eagerly
        torch.cuda.synchronize()
        if not torch.equal(got, out):
            raise RuntimeError("graph replay and eager step disagree")
        del g
    else:
        wall, gpu_ms = eager_wall, eager_gpu_ms

    # Region 2: the dominant kernel's own average duration: `steps` back-to-back launches of
    # it alone (pools cycled as in the steps) between one pair of HIP events on the stream the
    # kernel runs on. A pair of events around each single launch also holds that launch's
    # dispatch latency (a few microseconds); those per-launch brackets are kept for the spread.
    def phase1(i):
        kc, vc = pools[i % copies]
        if one_launch:
            pkv.paged_decode_into(q, kc, vc, bt, lens, case.scale, case.num_kv_heads, ps, 0, max_len, out, None,
                                  acc, m, l, counters, layout=case.layout)
        else:
            pkv.paged_decode_partial(q, kc, vc, bt, lens, case.scale, case.num_kv_heads, ps, max_len,
                                     acc, m, l, layout=case.layout)
    b_start, b_end = _events(2)
    torch.cuda.synchronize()
    b_start.record()
    for i in range(steps):
        phase1(i)
    b_end.record()
    torch.cuda.synchronize()
    avg_part_ms = b_start.elapsed_time(b_end) / steps
    evs = [_events(2) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    part_ms = sorted(a.elapsed_time(b) for a, b in evs)
    med_part_ms = part_ms[len(part_ms) // 2]

    kv_bytes = case.kv_bytes()
    return dict(
        copies=copies, pool_bytes=pool_bytes, kv_bytes=kv_bytes, graph=graph,
        wall_ms_per_step=wall * 1e3 / steps, gpu_ms_per_step=gpu_ms / steps,
        eager_wall_ms_per_step=eager_wall * 1e3 / steps, eager_gpu_ms_per_step=eager_gpu_ms / steps,
        partial_avg_ms=avg_part_ms, partial_median_ms=med_part_ms,
        partial_p10_ms=part_ms[len(part_ms) // 10], partial_p90_ms=part_ms[(9 * len(part_ms)) // 10],
    )


def bench_decode_fp8(case, steps, warmup):
    """The same batch with a float8 e4m3 cache (x-packed, x = 16) through paged_attention_v2,
    both phases per step, pools cycled as in bench_decode. KV bytes are one per element."""
    import torch
    import paged_kv_gqa_table_amd as pkv
    from paged_kv_gqa_table_amd import inputs
    dev = "cuda"
    k8, v8 = inputs.fp8_xpacked_pools(case)
    k8, v8 = k8.to(dev), v8.to(dev)
    pool_bytes = 2 * k8.numel()
    copies = max(1, min(8, math.ceil(3 * MALL_BYTES / max(1, pool_bytes))))
    pools = [(k8, v8)] + [(k8.clone(), v8.clone()) for _ in range(copies - 1)]
    q, bt, lens = case.query.to(dev), case.block_tables.to(dev), case.seq_lens.to(dev)
    S, H, D = case.num_seqs, case.num_heads, case.head_dim
    P = case.num_partitions(512)
    tmp = torch.empty((S, H, P, D), dtype=torch.float32, device=dev)
    es = torch.empty((S, H, P), dtype=torch.float32, device=dev)
    ml = torch.empty((S, H, P), dtype=torch.float32, device=dev)
    out = torch.empty((S, H, D), dtype=torch.bfloat16, device=dev)

    def step(i):
        kc, vc = pools[i % copies]
        pkv.paged_attention_v2(out, es, ml, tmp, q, kc, vc, case.num_kv_heads, case.scale, bt, lens,
                               case.block_size, case.max_seq_len, kv_cache_dtype="fp8", k_scale=1.0, v_scale=1.0)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    kv_bytes = int(case.seq_lens.sum()) * case.num_kv_heads * 2 * D
    return dict(ms=ms, kv_bytes=kv_bytes)


def read_ceiling(nbytes=1 << 30, reps=20):
    """Median bandwidth of the library's plain streaming read over a buffer 4x the size of
    the Infinity Cache (GB/s): the reference the paged gathers are compared with."""
    import torch
    import paged_kv_gqa_table_amd as pkv
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        pkv.read_bandwidth(buf, sink)
    evs = [_events(2) for _ in range(reps)]
    for a, b in evs:
        a.record()
        pkv.read_bandwidth(buf, sink)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    del buf
    torch.cuda.empty_cache()
    return nbytes / (ms[len(ms) // 2] * 1e-3) / 1e9


def bench_mla(case, steps, warmup):
    import torch
    import paged_kv_gqa_table_amd as pkv
    dev = "cuda"
    t = {k: getattr(case, k).to(dev) for k in ("q_nope", "q_pe", "ckv_cache", "kpe_cache", "qo_indptr",
                                                "kv_indptr", "kv_indices")}
    out = torch.empty_like(t["q_nope"])
    lse = torch.empty(t["q_nope"].shape[:2], dtype=torch.float32, device=dev)
    mql = case.max_q_len
    paged = case.kv_last_page_len is not None
    if paged:  # pages of several tokens: index scratch allocated once, outside the timing
        last = case.kv_last_page_len.to(dev)
        tok_indptr = torch.empty((case.batch + 1,), dtype=torch.int32, device=dev)
        tok_rows = torch.empty((case.kv_indices.numel() * case.page_size,), dtype=torch.int32, device=dev)

    def step():
        if paged:
            pkv.mla_paged_prefill_pages(t["q_nope"], t["q_pe"], t["ckv_cache"], t["kpe_cache"], t["qo_indptr"],
                                        t["kv_indptr"], t["kv_indices"], last, case.sm_scale, mql, tok_indptr,
                                        tok_rows, out, lse)
            return
        pkv.mla_paged_prefill(t["q_nope"], t["q_pe"], t["ckv_cache"], t["kpe_cache"], t["qo_indptr"],
                              t["kv_indptr"], t["kv_indices"], case.sm_scale, max_q_len=mql, out=out, lse=lse)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [_events(2) for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        step()
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    avg = sum(ms) / len(ms)
    # cold: before each timed launch, a 1 GiB buffer is rewritten (outside the events), which
    # evicts the pools from L2 and the Infinity Cache, so every key starts in HBM
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cold_evs = [_events(2) for _ in range(steps)]
    for i in range(steps):
        flush.fill_(float(i))
        cold_evs[i][0].record()
        step()
        cold_evs[i][1].record()
    torch.cuda.synchronize()
    cold = sorted(a.elapsed_time(b) for a, b in cold_evs)
    cold_avg = sum(cold) / len(cold)
    del flush
    flops = 16 * case.visible_pairs() * 2 * (512 + 64 + 512)
    return dict(ms=avg, median_ms=ms[len(ms) // 2], flops=flops, tflops=flops / (avg * 1e-3) / 1e12,
                cold_ms=cold_avg, cold_tflops=flops / (cold_avg * 1e-3) / 1e12)


def bench_mla_decode(case, steps, warmup, split, fused=False):
    """Time the split-K MLA decode (both launches) on the prefill-shaped case's q_len-1 rows,
    pools cycled like the GQA decode bench so that the Infinity Cache does not hold the keys.
    The steps are timed as one HIP graph replay (``ms``); the mean of eager per-step event
    pairs is ``eager_ms``."""
    import torch
    import paged_kv_gqa_table_amd as pkv
    dev = "cuda"
    t = {k: getattr(case, k).to(dev) for k in ("q_nope", "q_pe", "ckv_cache", "kpe_cache", "kv_indptr",
                                                "kv_indices")}
    pool_bytes = t["ckv_cache"].numel() * 2 + t["kpe_cache"].numel() * 2
    copies = max(1, min(8, math.ceil(3 * MALL_BYTES / max(1, pool_bytes))))
    pools = [(t["ckv_cache"], t["kpe_cache"])] + [(t["ckv_cache"].clone(), t["kpe_cache"].clone())
                                                 for _ in range(copies - 1)]
    kvl = (case.kv_indptr[1:] - case.kv_indptr[:-1])
    max_kv = int(kvl.max().item())
    B, H = case.batch, 16
    if split is None:
        split = pkv.mla_decode_default_split(B, max_kv, case.kv_indices.numel(), dev, kv_lens=kvl.tolist())
    P = -(-max_kv // split)
    parts = (torch.empty((B, H, P, 512), dtype=torch.float32, device=dev),
             torch.empty((B, H, P), dtype=torch.float32, device=dev),
             torch.empty((B, H, P), dtype=torch.float32, device=dev))
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    counters = torch.zeros((B,), dtype=torch.int32, device=dev) if fused else None

    def step(i):
        ckv, kpe = pools[i % copies]
        pkv.mla_paged_decode(t["q_nope"], t["q_pe"], ckv, kpe, t["kv_indptr"], t["kv_indices"], case.sm_scale,
                             split_tokens=split, max_kv_len=max_kv, out=out, lse=lse, partials=parts,
                             counters=counters)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [_events(2) for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        step(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    eager_ms = sum(ms) / len(ms)
    # the steps as one HIP graph replay, as for the GQA decode (an eager event pair around each
    # step also holds the host's submission gap between the two launches); checked bit for bit
    # against an eager run of the graph's last step
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            step(i)
    g.replay()  # untimed: the first replay uploads the graph
    torch.cuda.synchronize()
    t_start, t_end = _events(2)
    t_start.record()
    g.replay()
    t_end.record()
    torch.cuda.synchronize()
    graph_ms = t_start.elapsed_time(t_end) / steps
    got, got_lse = out.clone(), lse.clone()
    step(steps - 1)
    torch.cuda.synchronize()
    if not (torch.equal(got, out) and torch.equal(got_lse, lse)):
        raise RuntimeError("MLA decode: graph replay and eager step disagree")
    del g
    return dict(ms=graph_ms, eager_ms=eager_ms, eager_median_ms=ms[len(ms) // 2], split=split)


def cpu_baseline_decode(case, budget_s):
    """The float64 oracle as it stands, timed on this host over whole sequences of the batch."""
    import numpy as np
    import oracle
    import torch
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = os.cpu_count() or 1
    threads = max(blas_threads, torch.get_num_threads())
    lens = case.seq_lens.numpy()
    done_bytes = 0
    done_seqs = 0
    passes = 0
    t0 = time.perf_counter()
    per_tok = case.num_kv_heads * 2 * case.head_dim * (2 if case.dtype == "bf16" else 4)
    # whole passes over the batch, one sequence at a time, until the time budget is spent
    while time.perf_counter() - t0 < budget_s:
        for b in range(case.num_seqs):
            idx = torch.tensor([b])
            oracle.decode(case.query[idx], case.key_cache, case.value_cache, case.layout,
                          case.block_tables[idx], case.seq_lens[idx], case.scale, case.num_kv_heads,
                          case.block_size)
            done_bytes += int(lens[b]) * per_tok
            done_seqs += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        passes += 1
    dt = time.perf_counter() - t0
    return {"value": done_bytes / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done_seqs} sequence decodes ({passes} pass(es) over the {case.num_seqs}-sequence batch, "
                      f"all {case.num_heads} heads each; float64 numpy oracle, {dt:.1f} s wall)",
            "seconds": round(dt, 2), "ms_per_step_equiv": dt * 1e3 * (case.kv_bytes() / max(done_bytes, 1))}


def traffic_profile_path(workload):
    return os.path.join(ROOT, "profiles", f"decode_partial_{workload}_hbm_counters.md")


def profiled_traffic(workload):
    """HBM bytes per phase-1 launch from the committed counter summary of this workload
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel of known size), or None when there is
    none or the kernel's sources have changed since the counters were read."""
    import hashlib
    path = traffic_profile_path(workload)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        k, sep, v = line.partition(":")
        if sep and k.strip() in ("traffic_bytes_per_launch", "kernel_sources_sha256", "kernel_sources"):
            fields[k.strip()] = v.strip()
    if len(fields) != 3:
        return None
    h = hashlib.sha256()
    for name in fields["kernel_sources"].split():
        path = os.path.join(ROOT, "paged_kv_gqa_table_amd", "csrc", name)
        if not os.path.exists(path):
            return None
        with open(path, "rb") as f:
            h.update(f.read())
    if h.hexdigest() != fields["kernel_sources_sha256"]:
        return None
    return int(fields["traffic_bytes_per_launch"])


def calibrate_copy(mib):
    """A copy kernel of known size: dst = -src over `mib` MiB of float32, five launches.
    Each launch reads exactly mib MiB and writes exactly mib MiB of HBM (both far larger
    than the 256 MB Infinity Cache), which fixes the scale of FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib * 2**20 // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4,
                      "launches": 5}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              f"(each GPU would run its own share of sequences with no exchange).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy > 0:
        calibrate_copy(args.calibrate_copy)
        return
    from paged_kv_gqa_table_amd import inputs
    import paged_kv_gqa_table_amd as pkv
    pkv.lib()  # fail loudly if the HIP library is missing

    result = {}
    if args.workload == "mla_decode_b64":
        case = inputs.mla_decode_b64()
        r = bench_mla_decode(case, args.steps, args.warmup, split=None, fused=False)
        r2 = None if args.no_extra else bench_mla_decode(case, args.steps, args.warmup, split=None, fused=True)
        kv_b = sum(case.kv_lens()) * (512 + 64) * 2
        gbs = kv_b / (r["ms"] * 1e-3) / 1e9
        result = {
            "metric": "MLA decode ckv+kpe HBM GB/s and us per decode step (both launches), 1x MI355X",
            "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": r["ms"], "eager_us_per_step": r["eager_ms"] * 1e3, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": case.name, "batch": case.batch, "split_tokens": r["split"],
                       "kv_bytes_per_step": kv_b},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None},
            "one_launch_us": None if r2 is None else r2["ms"] * 1e3,
        }
        print(json.dumps(result), flush=True)
        return
    if args.workload == "mla_prefill_b8":
        case = inputs.mla_prefill_b8()
        r = bench_mla(case, args.steps, args.warmup)
        result = {
            "metric": "MLA causal paged prefill TFLOP/s (causal-visible flops) and us per prefill, 1x MI355X",
            "value": r["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": r["ms"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": case.name, "batch": case.batch, "total_q": case.total_q,
                       "num_pages": case.num_pages},
            "roofline": {"bound": "mfma", "achieved": r["tflops"], "peak": BF16_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": r["tflops"] / BF16_MFMA_PEAK_TFLOPS, "traffic": None},
            "cold_cache": {"us": r["cold_ms"] * 1e3, "TFLOP_s": r["cold_tflops"],
                           "frac_of_bf16_mfma_peak": r["cold_tflops"] / BF16_MFMA_PEAK_TFLOPS,
                           "note": "L2 and Infinity Cache flushed by a 1 GiB write before each timed launch"},
        }
        print(json.dumps(result), flush=True)
        return

    _log(f"generating workload {args.workload}")
    case = inputs.decode_workload(args.workload)
    r = bench_decode(case, args.steps, args.warmup, args.copies, graph=not args.eager)
    kv = r["kv_bytes"]
    ms = r["wall_ms_per_step"]
    gbs = kv / (ms * 1e-3) / 1e9
    achieved = kv / (r["partial_avg_ms"] * 1e-3) / 1e9
    result = {
        "metric": "achieved KV-cache HBM GB/s (% of peak) and us per decode step, 1x MI355X",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "us_per_step": ms * 1e3, "pct_of_peak": 100.0 * gbs / HBM_PEAK_GBS,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": case.dtype, "data": "synthetic",
        "config": {"workload": case.name, "num_seqs": case.num_seqs, "num_heads": case.num_heads,
                   "num_kv_heads": case.num_kv_heads, "head_dim": case.head_dim,
                   "block_size": case.block_size, "partition_size": case.partition_size,
                   "layout": case.layout, "kv_bytes_per_step": kv, "pool_copies_cycled": r["copies"],
                   "seq_len_total": int(case.seq_lens.sum()),
                   "submission": "hip_graph" if r["graph"] else "eager"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": profiled_traffic(args.workload),
                     "algorithmic_bytes_per_launch": kv,
                     "kernel": "paged_decode_partial", "kernel_avg_us": r["partial_avg_ms"] * 1e3,
                     "kernel_avg_method": f"one HIP event pair around {args.steps} back-to-back launches",
                     "launch_bracket_median_us": r["partial_median_ms"] * 1e3,
                     "launch_bracket_p10_us": r["partial_p10_ms"] * 1e3,
                     "launch_bracket_p90_us": r["partial_p90_ms"] * 1e3},
        "gpu_event_ms_per_step": r["gpu_ms_per_step"],
        "eager_us_per_step": r["eager_wall_ms_per_step"] * 1e3,
        "eager_gpu_event_us_per_step": r["eager_gpu_ms_per_step"] * 1e3,
    }
    if r["graph"]:
        result["graph_note"] = (f"the {args.steps} steps are captured once into a HIP graph and timed as one replay, "
                                "after the warmup steps and one untimed replay; its output equals an eager step "
                                "bit for bit")
    # warm reference: one pool only, so part of the KV stays in the Infinity Cache between steps
    rw = bench_decode(case, max(20, args.steps // 4), 5, copies=1, graph=not args.eager)
    result["warm_single_pool"] = {"us_per_step": rw["wall_ms_per_step"] * 1e3,
                                  "GB_s": kv / (rw["wall_ms_per_step"] * 1e-3) / 1e9,
                                  "kernel_avg_us": rw["partial_avg_ms"] * 1e3}
    ceiling = read_ceiling()
    result["roofline"]["measured_read_ceiling_GB_s"] = ceiling
    result["roofline"]["frac_of_measured_read_ceiling"] = achieved / ceiling
    if not args.no_extra and args.workload == "llama_gqa4":
        extra = {}
        rf = bench_decode_fp8(case, max(20, args.steps // 2), 5)
        extra["llama_gqa4_fp8_cache_v2"] = {
            "us_per_step": rf["ms"] * 1e3, "kv_bytes": rf["kv_bytes"],
            "GB_s": rf["kv_bytes"] / (rf["ms"] * 1e-3) / 1e9,
            "kernel": "paged_attention_v2 (float8 e4m3 x-packed cache, both phases)"}
        ro = bench_decode(case, max(20, args.steps // 2), 5, one_launch=True, graph=not args.eager)
        extra["llama_gqa4_one_launch"] = {"us_per_step": ro["wall_ms_per_step"] * 1e3,
                                          "GB_s": kv / (ro["wall_ms_per_step"] * 1e-3) / 1e9,
                                          "kernel_avg_us": ro["partial_avg_ms"] * 1e3}
        # the same lengths over 32-token blocks: the generic-block-size kernel
        c32 = inputs.make_decode(case.seq_lens.numpy(), case.num_heads, case.num_kv_heads, case.head_dim,
                                 dtype=case.dtype, layout=case.layout, block_size=32, seed=5,
                                 partition_size=case.partition_size, name="llama_gqa4_block32")
        r32 = bench_decode(c32, 20, 3, graph=not args.eager)
        extra["llama_gqa4_block32"] = {"us_per_step": r32["wall_ms_per_step"] * 1e3,
                                       "GB_s": r32["kv_bytes"] / (r32["wall_ms_per_step"] * 1e-3) / 1e9,
                                       "kernel": "generic-block-size kernel (32-token blocks), both phases"}
        del c32
        secondary = {}
        for name in ("wide_gqa6", "skewed_gqa8"):
            _log(f"secondary workload {name}")
            c2 = inputs.decode_workload(name)
            n2 = max(20, min(args.steps, 40))
            r2 = bench_decode(c2, n2, 5, graph=not args.eager)
            kv2 = c2.kv_bytes()
            ach2 = kv2 / (r2["partial_avg_ms"] * 1e-3) / 1e9
            line = {"steps": n2, "us_per_step": r2["wall_ms_per_step"] * 1e3,
                    "GB_s": kv2 / (r2["wall_ms_per_step"] * 1e-3) / 1e9,
                    "eager_us_per_step": r2["eager_wall_ms_per_step"] * 1e3,
                    "layout": c2.layout, "kv_bytes_per_step": kv2,
                    "roofline": {"bound": "hbm", "achieved": ach2, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": ach2 / HBM_PEAK_GBS, "traffic": profiled_traffic(name),
                                 "algorithmic_bytes_per_launch": kv2, "kernel": "paged_decode_partial",
                                 "kernel_avg_us": r2["partial_avg_ms"] * 1e3}}
            line["pct_of_peak"] = 100.0 * line["GB_s"] / HBM_PEAK_GBS
            r3 = bench_decode(c2, n2, 5, one_launch=True, graph=not args.eager)
            line["one_launch_us_per_step"] = r3["wall_ms_per_step"] * 1e3
            line["one_launch_GB_s"] = kv2 / (r3["wall_ms_per_step"] * 1e-3) / 1e9
            secondary[name] = line
            del c2
            torch.cuda.empty_cache()
        result["secondary"] = secondary
        try:
            _log("secondary workload mla_prefill_b8")
            mc = inputs.mla_prefill_b8()
            rm = bench_mla(mc, 20, 3)
            extra["mla_prefill_b8"] = {"us": rm["ms"] * 1e3, "TFLOP_s": rm["tflops"],
                                       "frac_of_bf16_mfma_peak": rm["tflops"] / BF16_MFMA_PEAK_TFLOPS,
                                       "cold_cache_us": rm["cold_ms"] * 1e3,
                                       "cold_cache_frac_of_bf16_mfma_peak": rm["cold_tflops"] / BF16_MFMA_PEAK_TFLOPS}
            del mc
            mp = inputs.mla_prefill_b8_pages(16)
            rp = bench_mla(mp, 20, 3)
            extra["mla_prefill_b8_pages16"] = {"us": rp["ms"] * 1e3, "TFLOP_s": rp["tflops"],
                                               "frac_of_bf16_mfma_peak": rp["tflops"] / BF16_MFMA_PEAK_TFLOPS}
            del mp
            md = inputs.mla_decode_b64()
            rd = bench_mla(md, 20, 3)
            kv_b = sum(md.kv_lens()) * (512 + 64) * 2  # ckv + kpe bytes of every key, read once
            extra["mla_decode_b64_prefill_kernel"] = {
                "us": rd["ms"] * 1e3, "kv_GB_s": kv_b / (rd["ms"] * 1e-3) / 1e9,
                "frac_of_hbm_peak": kv_b / (rd["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, "kernel": "mla_paged_prefill (q_len 1)"}
            rs = bench_mla_decode(md, 50, 5, split=None, fused=False)
            rs2 = bench_mla_decode(md, 50, 5, split=None, fused=True)
            extra["mla_decode_b64"] = {"us": rs["ms"] * 1e3, "kv_GB_s": kv_b / (rs["ms"] * 1e-3) / 1e9,
                                       "frac_of_hbm_peak": kv_b / (rs["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                       "split_tokens": rs["split"], "one_launch_us": rs2["ms"] * 1e3,
                                       "eager_us": rs["eager_ms"] * 1e3, "one_launch_eager_us": rs2["eager_ms"] * 1e3,
                                       "timing": "one HIP graph replay of 50 steps (eager per-step events beside)",
                                       "kernel": "mla_paged_decode (split-K, default splits, both launches)"}
        except NotImplementedError as e:
            extra["mla_prefill_b8"] = {"error": str(e)}
        result["extra"] = extra
    if not args.no_cpu:
        _log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline_decode(case, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
