#!/usr/bin/env python3
"""Benchmark of the paged KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gqa|long|prefix_cow|mixed|spec|swap]
                    [--layout paged|contiguous] [--block-size 8|16|32] [--shared-prefix]
                    [--spec-path multi_query|prefill] [--no-cpu-baseline] [--no-read-ceiling]

One step is one pass of the path over one synthetic batch: the step's cache
write (paged_kv_write) followed by paged decode attention (split-context
partitions + log-sum-exp merge); the prefix workload adds its copy-on-write
block copies and the mixed workload its chunked-prefill attention.  Inputs are
resident in HBM before timing starts.  Several device copies of the pools are
rotated step by step so that repeated steps cannot be served from the 256 MB
Infinity Cache.

Prints ONE JSON line: metric/value = decode KV GB/s of the whole step
(algorithmic KV bytes: K and V of every valid token, read once per
(sequence, kv head)), plus seqs/s, a roofline object for the decode kernels
(HIP events on the launch stream; also per-call p10/p50/p90 and the fraction of
the measured streaming-read ceiling of a 4 GiB buffer), the device time of the
step's write and block-copy calls, and the CPU oracle timed on this host.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
METRIC = "paged decode attention KV GB/s (% of HBM peak) + seqs/s, 1xMI355X"


def kv_bytes(context_lens, num_kv_heads, head_dim, elem) -> int:
    """Algorithmic bytes of one decode call: K and V of every valid token, each read
    once per (sequence, kv head) -- 2*N*L*H*D*P of the vAttention page with N = 1."""
    return int(2 * np.asarray(context_lens, dtype=np.int64).sum() * num_kv_heads * head_dim * elem)


def shared_kv_bytes(context_lens, prefix_len, num_kv_heads, head_dim, elem) -> int:
    """Algorithmic bytes of a decode whose sequences all share their first prefix_len
    tokens: the prefix K/V once per kv head, then each sequence's own tokens."""
    own = np.asarray(context_lens, dtype=np.int64) - prefix_len
    return int(2 * (prefix_len + own.sum()) * num_kv_heads * head_dim * elem)


def prefill_flops(pre) -> int:
    """Algorithmic flops of causal chunk attention: 4*D per visible (query, key) pair
    per query head (QK^T and PV)."""
    tot = 0
    for c in range(pre.num_chunks):
        nq = int(pre.cu_q_lens[c + 1] - pre.cu_q_lens[c])
        n = int(pre.context_lens[c])
        visible = nq * (n - nq) + nq * (nq + 1) // 2
        tot += visible
    return int(4 * pre.head_dim * pre.num_q_heads * tot)


def recorded_traffic(workload_name, prefix="decode_"):
    """Counter-derived HBM bytes per call of the timed kernels, as recorded under profiles/
    with the hashes of the sources they were measured on; None when absent or stale."""
    import hashlib
    stem = prefix + workload_name.replace("_decode", "")
    path = os.path.join(ROOT, "profiles", f"{stem}_traffic.json")
    try:
        rec = json.load(open(path))
        for name, sha in rec["sources_sha256"].items():
            src = os.path.join(ROOT, "paged_kv_cache_79_amd", "csrc", name)
            if hashlib.sha256(open(src, "rb").read()).hexdigest() != sha:
                return None
    except (OSError, ValueError, KeyError):
        return None
    return rec["traffic_bytes_per_call"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# CPU oracle baseline (bounded sample, on this host's cores)
# ----------------------------------------------------------------------------
# Batches the oracle workers read, by leg name: set before the worker pool is forked
# (which happens before this process first touches the GPU), so every worker inherits
# them and no worker inherits a GPU context.
_ORACLE_BATCHES = {}
# The box gives one GPU's job a share of 16 host cores, whatever the affinity mask shows.
CPU_SHARE = 16


def _oracle_unit(task):
    from threadpoolctl import threadpool_limits
    from oracle import paged as O
    name, s = task
    b, k, v = _ORACLE_BATCHES[name]
    with threadpool_limits(1):
        O.decode(b.q, k, v, b.block_tables, b.context_lens, b.scale, b.dtype, b.num_kv_heads,
                 seqs=[s])
    return s


def oracle_register(name, b):
    """The oracle's view of a decode batch after the step's cache write."""
    from oracle import paged as O
    k = O.kv_write(b.k_pool, b.k_new, b.slot_mapping)
    v = O.kv_write(b.v_pool, b.v_new, b.slot_mapping)
    _ORACLE_BATCHES[name] = (b, k, v)


def oracle_pool():
    """Worker processes for the oracle baseline, one per core of this job's share."""
    import multiprocessing as mp
    avail = len(os.sched_getaffinity(0))
    used = max(1, min(avail, CPU_SHARE))
    return mp.get_context("fork").Pool(used), avail, used


def cpu_baseline(pool, avail, used, name, target_cpu_s=20.0):
    """Time the oracle's decode of the batch registered as `name` on this host: one
    sequence per task over the worker pool, whole passes over the batch repeated until
    about target_cpu_s of CPU work (wall time x workers)."""
    b = _ORACLE_BATCHES[name][0]
    units = [(name, s) for s in range(b.num_seqs)]
    # an untimed pass warms the workers up; the first timed pass sizes the sample:
    # whole passes until about target_cpu_s
    pool.map(_oracle_unit, units, chunksize=1)
    t0 = time.perf_counter()
    pool.map(_oracle_unit, units, chunksize=1)
    first = time.perf_counter() - t0
    passes = max(1, min(64, int(round(target_cpu_s / max(first * used, 1e-3)))))
    for _ in range(passes - 1):
        pool.map(_oracle_unit, units, chunksize=1)
    wall = time.perf_counter() - t0
    byts = passes * kv_bytes(b.context_lens, b.num_kv_heads, b.head_dim, 2 if b.dtype == "bf16" else 4)
    return {"value": round(byts / wall / 1e9, 4), "unit": "GB/s", "cores": used,
            "cores_available": avail, "kind": "oracle",
            "seqs_per_s": round(passes * b.num_seqs / wall, 2), "wall_s": round(wall, 2),
            "cpu_s": round(wall * used, 1),
            "sample": f"{passes} pass(es) of fp64 numpy decode over all {b.num_seqs} sequences of "
                      f"the {b.name} batch, one sequence per task on {used} worker processes "
                      f"({avail} cores in the affinity mask, {CPU_SHARE} the job's share)"}


# ----------------------------------------------------------------------------
# GPU
# ----------------------------------------------------------------------------
def read_ceiling(buffer_bytes=4 << 30, waves=8192, reps=5):
    """Measured streaming-read ceiling: pkv_bench_read (libpkvbench.so) over a buffer
    16x the 256 MB Infinity Cache; median GB/s of 3 runs of `reps` passes."""
    import ctypes
    import torch
    import paged_kv_cache_79_amd as pkv
    path = os.path.join(os.path.dirname(pkv.LIB_PATH), "libpkvbench.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    lib.pkv_bench_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_int32, ctypes.c_void_p]
    lib.pkv_bench_read.restype = ctypes.c_int
    buf = torch.ones(buffer_bytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(waves * 64, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def once():
        rc = lib.pkv_bench_read(buf.data_ptr(), buffer_bytes, sink.data_ptr(), waves,
                                stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"pkv_bench_read failed: {rc}")

    once()
    runs = []
    for _ in range(3):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(reps):
            once()
        t1.record(stream)
        torch.cuda.synchronize()
        runs.append(buffer_bytes * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9)
    del buf, sink
    return sorted(runs)[1]


def device_us(fn, n, busy, stream):
    """Device time per call of a short call: the n calls are enqueued while the stream
    is still busy with `busy` (long work issued first), so the events measure the
    device, not the host's call rate."""
    import torch
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    busy()
    t0.record(stream)
    for i in range(n):
        fn(i)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / n


def per_call_us(fn, n, stream):
    """Each of n calls bracketed by its own pair of events: (p10, p50, p90) in us."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fn(i)
        b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    return [round(float(x), 2) for x in np.percentile(t, [10, 50, 90])]

def _dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def make_workload(name, block_size=16, contiguous=False, num_seqs=4096):
    import workloads as W
    if contiguous and name not in ("gqa", "long"):
        raise SystemExit("--layout contiguous applies to the gqa and long workloads")
    if block_size != 16 and name not in ("gqa", "long"):
        raise SystemExit("--block-size applies to the gqa and long workloads")
    if name == "gqa":
        b = W.gqa(poison=False, block_size=block_size, contiguous=contiguous)
        return dict(batch=b, extra=None, prefill=None)
    if name == "long":
        return dict(batch=W.long_context(poison=False, block_size=block_size, contiguous=contiguous),
                    extra=None, prefill=None)
    if name == "prefix_cow":
        p = W.prefix_cow(poison=False)
        return dict(batch=p.batch, extra=p, prefill=None)
    if name == "mixed":
        m = W.mixed(poison=False)
        return dict(batch=m.decode, extra=m, prefill=m.prefill)
    if name == "many":
        # the GQA geometry with many short sequences (U[64, 512] tokens): the merge's
        # cost per output row, independent of the number of sequences
        rng = np.random.Generator(np.random.PCG64(79010 + num_seqs))
        ctx = rng.integers(64, 512, size=num_seqs, endpoint=True)
        b = W.build_decode_batch(name=f"many_{num_seqs}_bf16", dtype="bf16", context_lens=ctx,
                                 num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                                 seed=79010 + num_seqs, poison=False)
        return dict(batch=b, extra=None, prefill=None)
    raise SystemExit(f"unknown workload {name}")


def run_spec(args):
    """Speculative-decode verification: each sequence writes its k + 1 newest tokens and
    attends with k + 1 causal queries (paged_kv_write + paged_attention_prefill_chunk)."""
    import torch
    import paged_kv_cache_79_amd as pkv
    import workloads as W
    log("building workload spec")
    sb = W.spec_decode(poison=False, block_size=args.block_size, draft=args.draft)
    pre = sb.prefill
    nq = sb.draft + 1
    pool_bytes = 2 * sb.k_pool.nbytes
    copies = max(2, min(8, int(math.ceil(2.4e9 / max(pool_bytes, 1)))))
    k0, v0 = _dev(sb.k_pool), _dev(sb.v_pool)
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]
    q, cu = _dev(pre.q), _dev(pre.cu_q_lens)
    tab, ctx = _dev(pre.block_tables), _dev(pre.context_lens)
    k_new, v_new, slots = _dev(sb.k_new), _dev(sb.v_new), _dev(sb.slot_mapping)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    mq = args.spec_path == "multi_query"
    pws = None
    if not mq and not args.no_prefill_split:
        pws = torch.empty(max(1, pkv.paged_attention_prefill_chunk_workspace_bytes(
            pre.num_q_heads, pre.num_kv_heads, pre.head_dim)), dtype=torch.uint8, device="cuda")
    if mq:
        ws = pkv.decode_workspace(pkv.paged_attention_decode_multi_query_workspace_bytes(
            pre.num_chunks, nq, pre.num_q_heads, pre.num_kv_heads, pre.head_dim), q.device)

    def attend(i):
        kp, vp = pools[i % copies]
        if mq:
            pkv.paged_attention_decode_multi_query(out, q, kp, vp, tab, ctx, nq,
                                                   pre.max_context_len, pre.scale, workspace=ws)
        else:
            pkv.paged_attention_prefill_chunk(out, q, cu, kp, vp, tab, ctx, nq,
                                              pre.max_context_len, pre.scale, workspace=pws,
                                              split=pws is not None)

    def step(i):
        kp, vp = pools[i % copies]
        pkv.paged_kv_write(kp, vp, k_new, v_new, slots)
        attend(i)

    def timed(fn, n):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(n):
            fn(i)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n

    for i in range(args.warmup):
        step(i)
    ms_step = timed(step, args.steps)
    runs = [timed(attend, args.steps) for _ in range(3)]
    att = sorted(runs)[1]
    byts = kv_bytes(pre.context_lens, pre.num_kv_heads, pre.head_dim, 2)
    value = byts / (ms_step * 1e-3) / 1e9
    achieved = byts / (att * 1e-3) / 1e9
    return {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "spec_decode_bf16", "num_seqs": pre.num_chunks,
                   "queries_per_seq": nq, "num_q_heads": pre.num_q_heads,
                   "num_kv_heads": pre.num_kv_heads, "head_dim": pre.head_dim,
                   "block_size": pre.block_size, "max_context_len": pre.max_context_len,
                   "mean_context_len": round(float(np.mean(pre.context_lens)), 1),
                   "path": args.spec_path, "pool_copies_rotated": copies},
        "seqs_per_s": round(pre.num_chunks / (ms_step * 1e-3), 1),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "kv_bytes_per_step": byts,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     # the counters were taken on the default batch (block 16, 3 drafts)
                     "traffic": recorded_traffic("spec")
                     if mq and pre.block_size == 16 and sb.draft == 3 else None,
                     "kernel": ("paged_attention_decode_multi_query (attention kernel + merge "
                                "kernel)" if mq else
                                "paged_attention_prefill_chunk with k + 1 queries per sequence"),
                     "avg_us": round(att * 1e3, 2), "runs_us": [round(x * 1e3, 2) for x in runs]},
        "cpu_baseline": None,
    }


def run_swap(args):
    """Preemption by swapping: 2048 blocks of the GQA geometry (8 kv heads x 16 tokens x
    D 128, bf16; 64 KiB of K+V per block) copied device -> pinned host -> device, with
    scattered device ids (one DMA copy per block) and with contiguous runs."""
    import torch
    import paged_kv_cache_79_amd as pkv
    nb_dev, n, hkv, bs, d = 16384, 2048, 8, 16, 128
    k = torch.randn((nb_dev, hkv, bs, d), device="cuda").to(torch.bfloat16)
    v = torch.randn((nb_dev, hkv, bs, d), device="cuda").to(torch.bfloat16)
    hk = torch.empty((n, hkv, bs, d), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    rng = np.random.Generator(np.random.PCG64(79007))
    scattered = rng.choice(nb_dev, n, replace=False)
    maps = {"scattered": scattered, "runs": np.arange(n) + 4096}
    stream = torch.cuda.current_stream()
    byts = 2 * n * hkv * bs * d * 2
    res = {}
    for name, ids in maps.items():
        out_map = np.stack([ids, np.arange(n)], axis=1)
        in_map = np.stack([np.arange(n), ids], axis=1)
        for direction, (dk, dv, sk, sv, mp) in {"out": (hk, hv, k, v, out_map),
                                               "in": (k, v, hk, hv, in_map)}.items():
            pkv.swap_blocks(dk, dv, sk, sv, mp)
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            h0 = time.perf_counter()
            t0.record(stream)
            reps = max(2, args.steps // 10)
            for _ in range(reps):
                pkv.swap_blocks(dk, dv, sk, sv, mp)
            t1.record(stream)
            host_s = (time.perf_counter() - h0) / reps
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1) / reps
            res[f"{name}_{direction}"] = {"ms": round(ms, 4), "GB/s": round(byts / (ms * 1e-3) / 1e9, 2),
                                          "host_enqueue_ms": round(host_s * 1e3, 3)}
    best = max(r["GB/s"] for r in res.values())
    return {"metric": "swap_blocks GB/s (device <-> pinned host), 1xMI355X", "value": best,
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": res["scattered_out"]["ms"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "swap", "blocks": n, "bytes_per_direction": byts,
                       "block_bytes_kv": 2 * hkv * bs * d * 2},
            "swap": res, "roofline": None, "cpu_baseline": None}


# The default run: the GQA batch (the headline line), the long-context shard and the
# mixed chunked-prefill + decode batch, each a leg of the same JSON line.
DEFAULT_LEGS = ("gqa", "long", "mixed")


def prepare(name, args):
    """Host-side workload of one leg (numpy only: nothing here touches the GPU)."""
    log(f"building workload {name}")
    contig = args.layout == "contiguous"
    wl = make_workload(name, args.block_size, contig, args.num_seqs)
    b = wl["batch"]
    log(f"workload ready: {b.num_seqs} sequences, max context {b.max_context_len}")
    return dict(name=name, wl=wl, contig=contig)


def gpu_leg(prep, args, ceiling):
    """Time one leg on the GPU: the whole step, the decode call alone (roofline), per-call
    percentiles, the step's other calls and, for the mixed batch, the prefill call."""
    import torch
    import paged_kv_cache_79_amd as pkv

    wl, contig, name = prep["wl"], prep["contig"], prep["name"]
    b = wl["batch"]
    elem = 2 if b.dtype == "bf16" else 4
    if contig:
        # the unpaged baseline: the same K/V values in [S][L][Hkv][D] slabs, already
        # holding the step's new token (no cache write is timed)
        kc, vc = b.extra["k_cache"], b.extra["v_cache"]
        pool_bytes = 2 * kc.nbytes
    else:
        pool_bytes = 2 * b.k_pool.nbytes
    # enough pool copies that a rotation cycle spans well over 4x the 256 MB MALL
    copies = max(2, min(8, int(math.ceil(2.4e9 / max(pool_bytes, 1)))))
    k0, v0 = (_dev(kc), _dev(vc)) if contig else (_dev(b.k_pool), _dev(b.v_pool))
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]
    q = _dev(b.q)
    tables = _dev(b.block_tables)
    ctx = _dev(b.context_lens)
    k_new, v_new, slots = _dev(b.k_new), _dev(b.v_new), _dev(b.slot_mapping)
    out = torch.empty_like(q)
    pt = args.partition_tokens            # 0: balanced split over the resident waves
    ws_bytes = pkv.paged_attention_decode_workspace_bytes(b.num_seqs, b.num_q_heads, b.num_kv_heads,
                                                          b.head_dim, b.max_context_len, pt)
    extra = wl["extra"]
    cow_map = _dev(extra.block_mapping) if name == "prefix_cow" else None
    shared = None
    if args.shared_prefix:
        if name != "prefix_cow" or pt != 0:
            raise SystemExit("--shared-prefix applies to the prefix_cow workload (balanced split)")
        # one group of every sequence; the blocks still shared after copy-on-write
        plen = (len(extra.prefix_blocks) - 1) * b.block_size
        S = b.num_seqs
        shared = dict(plen=plen, seq_prefix=_dev(np.full(S, plen, np.int32)),
                      first=_dev(np.array([0], np.int32)), num=_dev(np.array([S], np.int32)),
                      pre=_dev(np.array([plen], np.int32)))
        ws_bytes = pkv.paged_attention_decode_shared_prefix_workspace_bytes(
            b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim, b.max_context_len, plen)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    pre = wl["prefill"]
    if pre is not None:
        pq, pcu = _dev(pre.q), _dev(pre.cu_q_lens)
        ptab, pctx = _dev(pre.block_tables), _dev(pre.context_lens)
        pout = torch.empty_like(pq)
        # the prefill's workspace lets it split uneven chunks over keys (--no-prefill-split: none)
        pws = None
        if not args.no_prefill_split:
            pws = torch.zeros(max(1, pkv.paged_attention_prefill_chunk_workspace_bytes(
                pre.num_q_heads, pre.num_kv_heads, pre.head_dim)), dtype=torch.uint8, device="cuda")

    stream = torch.cuda.current_stream()

    def decode(i):
        kp, vp = pools[i % copies]
        if contig:
            pkv.contiguous_attention_decode(out, q, kp, vp, ctx, b.max_context_len, b.scale,
                                            workspace=ws)
            return
        if shared is not None:
            pkv.paged_attention_decode_shared_prefix(
                out, q, kp, vp, tables, ctx, b.max_context_len, b.scale, shared["seq_prefix"],
                shared["first"], shared["num"], shared["pre"], b.num_seqs, shared["plen"],
                workspace=ws)
            return
        pkv.paged_attention_decode(out, q, kp, vp, tables, ctx, b.max_context_len, b.scale,
                                   partition_tokens=pt, workspace=ws)

    def prefill(i):
        kp, vp = pools[i % copies]
        pkv.paged_attention_prefill_chunk(pout, pq, pcu, kp, vp, ptab, pctx, pre.max_q_len,
                                          pre.max_context_len, pre.scale, workspace=pws,
                                          split=pws is not None)

    def step(i):
        if contig:
            decode(i)
            return
        kp, vp = pools[i % copies]
        if cow_map is not None:
            pkv.copy_blocks(kp, vp, cow_map)
        pkv.paged_kv_write(kp, vp, k_new, v_new, slots)
        if pre is not None:
            prefill(i)
        decode(i)

    def timed(fn, n):
        """HIP events on the launch stream around n back-to-back calls; mean ms per call."""
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(n):
            fn(i)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n

    log(f"{name}: {copies} pool copies on device; warmup {args.warmup}, timing {args.steps} steps")
    for i in range(args.warmup):
        step(i)
    ms_step = timed(step, args.steps)
    # the decode call alone, same inputs and pool rotation, for the roofline
    dec_runs = [timed(decode, args.steps) for _ in range(3)]
    dec_avg = sorted(dec_runs)[1]
    dec_pct = per_call_us(decode, args.steps, stream)
    # the step's other calls alone (device time: enqueued behind 8 decode calls)
    parts = {}
    if not contig:
        def busy():
            for i in range(8):
                decode(i)

        def write(i):
            kp, vp = pools[i % copies]
            pkv.paged_kv_write(kp, vp, k_new, v_new, slots)
        parts["paged_kv_write_us"] = round(device_us(write, 10, busy, stream), 2)
        if cow_map is not None:
            def copy(i):
                kp, vp = pools[i % copies]
                pkv.copy_blocks(kp, vp, cow_map)
            parts["copy_blocks_us"] = round(device_us(copy, 10, busy, stream), 2)
    byts = kv_bytes(b.context_lens, b.num_kv_heads, b.head_dim, elem)
    value = byts / (ms_step * 1e-3) / 1e9
    # the roofline counts what the path has to read: with a shared prefix its K/V once
    # per kv head, plus every sequence's own tokens
    unique = byts if shared is None else shared_kv_bytes(b.context_lens, shared["plen"],
                                                         b.num_kv_heads, b.head_dim, elem)
    achieved = unique / (dec_avg * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b.dtype,
        "data": "synthetic",
        "config": {"workload": b.name, "num_seqs": b.num_seqs, "num_q_heads": b.num_q_heads,
                   "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim,
                   "block_size": b.block_size, "max_context_len": b.max_context_len,
                   "mean_context_len": round(float(np.mean(b.context_lens)), 1),
                   "split": "balanced" if pt == 0 else f"partitions of {pt}",
                   "layout": "contiguous [S][L][Hkv][D], no block table (step = decode only)"
                             if contig else "paged [NB][Hkv][bs][D]",
                   "step": ("decode" if contig else
                            " + ".join((["copy_blocks"] if cow_map is not None else []) +
                                       ["paged_kv_write"] +
                                       (["paged_attention_prefill_chunk"] if pre is not None else []) +
                                       ["decode"])),
                   "pool_copies_rotated": copies,
                   **({"decode": f"shared prefix: one group of {b.num_seqs}, "
                                 f"{shared['plen']}-token prefix"} if shared else {})},
        "seqs_per_s": round(b.num_seqs / (ms_step * 1e-3), 1),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "kv_bytes_per_step": byts,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (recorded_traffic(("shared_prefix_" if shared else "") + b.name)
                                 if pt == 0 and not contig and args.block_size == 16 else None),
                     "kernel": ("contiguous_attention_decode" if contig else
                                "paged_attention_decode_shared_prefix (prefix pass + "
                                "attention kernel + merge kernel)" if shared else
                                "paged_attention_decode (whole call)"),
                     "algorithmic_bytes": unique,
                     "avg_us": round(dec_avg * 1e3, 2),
                     "runs_us": [round(x * 1e3, 2) for x in dec_runs],
                     "per_call_us_p10_p50_p90": dec_pct,
                     "read_ceiling_GBs": None if ceiling is None else round(ceiling, 1),
                     "frac_of_read_ceiling": None if ceiling is None
                                             else round(achieved / ceiling, 4)},
        **parts,
    }
    if pre is not None:
        # prefill alone, same inputs and pool rotation
        p_runs = [timed(prefill, max(5, args.steps // 2)) for _ in range(3)]
        p_ms = sorted(p_runs)[1]
        fl = prefill_flops(pre)
        tf = fl / (p_ms * 1e-3) / 1e12
        rec["prefill"] = {
            "config": {"chunks": pre.num_chunks, "queries_per_chunk": pre.max_q_len,
                       "max_context_len": pre.max_context_len, "causal": True},
            "avg_us": round(p_ms * 1e3, 2), "runs_us": [round(x * 1e3, 2) for x in p_runs],
            "flops": fl, "key_split_allowed": pws is not None,
            "tflops": round(tf, 2), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": recorded_traffic("prefill_mixed_bf16", prefix="")
                                    if pws is not None else None,
                         "kernel": "paged_attention_prefill_chunk (whole call)"}}
    log(f"{name}: {ms_step * 1e3:.1f} us/step, decode {dec_avg * 1e3:.1f} us"
        + (f", prefill {rec['prefill']['avg_us']:.1f} us" if pre is not None else ""))
    del pools, k0, v0, ws
    torch.cuda.empty_cache()
    return rec


def run(args):
    names = list(DEFAULT_LEGS) if args.workload == "all" else [args.workload]
    if args.layout == "contiguous" and len(names) > 1:
        raise SystemExit("--layout contiguous needs --workload gqa or long")
    preps = [prepare(n, args) for n in names]
    pool = None
    want_cpu = not args.no_cpu_baseline and args.layout != "contiguous"
    if want_cpu:
        for p in preps:
            oracle_register(p["name"], p["wl"]["batch"])
        # forked before the first GPU call, so no worker inherits a GPU context
        pool, avail, used = oracle_pool()
    try:
        ceiling = read_ceiling() if not args.no_read_ceiling else None
        recs = [gpu_leg(p, args, ceiling) for p in preps]
        for p, r in zip(preps, recs):
            if want_cpu:
                log(f"{p['name']}: timing the CPU oracle")
                r["cpu_baseline"] = cpu_baseline(pool, avail, used, p["name"])
            else:
                r["cpu_baseline"] = None
    finally:
        if pool is not None:
            pool.close()
            pool.join()
    top = recs[0]
    if len(recs) > 1:
        top["legs"] = {r["config"]["workload"]: r for r in recs[1:]}
    return top


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    choices=["all", "gqa", "long", "prefix_cow", "mixed", "spec", "swap", "many"],
                    help="all (default): the gqa line with the long and mixed batches as legs")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--num-seqs", type=int, default=4096,
                    help="many: number of sequences of U[64, 512] tokens")
    ap.add_argument("--layout", default="paged", choices=["paged", "contiguous"],
                    help="contiguous: the unpaged baseline on the same K/V values (gqa, long)")
    ap.add_argument("--block-size", type=int, default=16, choices=[8, 16, 32],
                    help="pool block size of the gqa and long workloads")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="prefix_cow: decode through the shared-prefix path (prefix read once)")
    ap.add_argument("--draft", type=int, default=3,
                    help="spec: draft tokens k per sequence (k + 1 queries each)")
    ap.add_argument("--spec-path", default="multi_query", choices=["multi_query", "prefill"],
                    help="spec: attention through the multi-query decode or chunked prefill")
    ap.add_argument("--no-prefill-split", action="store_true",
                    help="mixed, spec --spec-path prefill: chunked prefill without a workspace "
                         "(one workgroup per query tile)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the streaming-read ceiling measurement (4 GiB buffer)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    runners = {"spec": run_spec, "swap": run_swap}
    rec = runners.get(args.workload, run)(args)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
