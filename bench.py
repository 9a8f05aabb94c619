#!/usr/bin/env python3
"""Benchmark of the paged-attention decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]

One step is the device half of a decode step of the engine for a batch of
sequences: the new token's key/value of every sequence is written into its
cache slot, and attention runs from that token over the whole cached
context.  By default both happen in one launch (pa_decode_append; with
split-K the partials are merged inside the same launch); --unfused runs
pa_reshape_and_cache and pa_decode as two launches.  Host metadata (block
tables from the free_block_queue allocator, slot mapping, the decode work
plan) is built before timing, as the engine's CPU side does ahead of the
step, and its cost is reported separately: once from scratch, and as the
incremental per-step update (one more token per sequence).  The steps are
replayed from a captured HIP graph, as the pages' engine replays
pre-recorded graphs to cut launch overhead; the decode kernel's own duration
is timed the same way from a graph of its launches alone (HIP events around
the replays, on the stream the kernels run on).

Inputs are seeded synthetic draws (paged_attention_kv_block_amd.inputs) that
are resident in HBM before timing.  The default workload is the largest
decode batch, the long-context one: 16 sequences of 32K-131K tokens (uniform),
64/8 heads, head size 128, bf16, split-K over 1024-token partitions with the
log-sum-exp merge (a 5.4 GB pool).  --workload 1 is the TinyLlama-1.1B-shaped
batch (64 sequences, 32/4 heads, head size 64, lengths uniform in [128,
2048]); its pool (~79 MB) fits in the 256 MB Infinity Cache, so the step
rotates over enough identical pool copies (>= 768 MB) that each step reads
its pool from HBM, as a real model's next visit to the same layer would.
--workload 2 is the Llama-3-8B-shaped batch (256 sequences, split-K 512).

Prints one JSON line: metric/value (algorithmic GB/s of the whole step),
the HBM roofline of the dominant kernel (decode), and the fp64 CPU oracle
timed on this host as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
METRIC = "paged-attn decode KV GB/s (% of HBM peak) + context-tokens/s, 1 GPU"
TRAFFIC_FILES = {False: os.path.join(ROOT, "profiles", "decode_append_traffic.json"),
                 True: os.path.join(ROOT, "profiles", "decode_traffic.json")}
# counters of the fused decode launch of the larger workloads, at their own
# partition sizes
WORKLOAD_TRAFFIC = {2: os.path.join(ROOT, "profiles", "decode_append_traffic_llama3-8b.json"),
                    4: os.path.join(ROOT, "profiles", "decode_append_traffic_long-context.json")}
# the same over the FP8 cache (pa_decode_append_fp8, each workload's own
# partition size)
FP8_TRAFFIC = {1: os.path.join(ROOT, "profiles", "decode_append_fp8_traffic_tinyllama-1.1b.json"),
               2: os.path.join(ROOT, "profiles", "decode_append_fp8_traffic_llama3-8b.json"),
               4: os.path.join(ROOT, "profiles", "decode_append_fp8_traffic_long-context.json")}
VARLEN_TRAFFIC = os.path.join(ROOT, "profiles", "varlen_traffic.json")
MULTI_TRAFFIC = os.path.join(ROOT, "profiles", "decode_multi_traffic.json")
MULTI_FP8_TRAFFIC = os.path.join(ROOT, "profiles", "decode_multi_fp8_traffic.json")
PREFILL_TRAFFIC = os.path.join(ROOT, "profiles", "prefill_traffic.json")
PREFILL_SOURCES = ["paged_attention_kv_block_amd/csrc/pa_prefill.hip",
                   "paged_attention_kv_block_amd/csrc/pa_prefill_wide_dev.h",
                   "paged_attention_kv_block_amd/csrc/pa_common.h"]
VARLEN_SOURCES = ["paged_attention_kv_block_amd/csrc/pa_varlen.hip",
                  "paged_attention_kv_block_amd/csrc/pa_decode_dev.h",
                  "paged_attention_kv_block_amd/csrc/pa_prefill_wide_dev.h",
                  "paged_attention_kv_block_amd/csrc/pa_common.h"]
DECODE_SOURCES = ["paged_attention_kv_block_amd/csrc/pa_decode.hip",
                  "paged_attention_kv_block_amd/csrc/pa_decode_dev.h",
                  "paged_attention_kv_block_amd/csrc/pa_common.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def default_partition(wl) -> int:
    """The workload's own split-K partition if it names one, else 0 (one pass
    per sequence and KV head: the best measured for the TinyLlama-shaped
    batch, whose 256 (sequence, head) items already cover the 256 CUs)."""
    if wl.partition_size:
        return wl.partition_size
    return 0


def decode_bytes(wl, seq_lens, kv_bytes=None) -> int:
    """Algorithmic bytes of one decode launch: valid K/V of every context
    token, query in, output out, the used block-table entries, seq_lens.
    kv_bytes: bytes of a cached element when the cache is narrower than the
    queries (1 for FP8)."""
    db = wl.dtype_bytes
    kb = db if kv_bytes is None else kv_bytes
    n = len(seq_lens)
    kv = int(sum(int(L) for L in seq_lens)) * 2 * wl.num_kv_heads * wl.head_size * kb
    qo = 2 * n * wl.num_q_heads * wl.head_size * db
    bt = sum((int(L) + wl.block_size - 1) // wl.block_size for L in seq_lens) * 4
    return kv + qo + bt + 4 * n


def cache_write_bytes(wl, kv_bytes=None, num_seqs=None) -> int:
    """Writing one new token per sequence into the cache: read its K and V
    rows, write them (as kv_bytes-wide elements for an FP8 cache)."""
    row = wl.num_kv_heads * wl.head_size * wl.dtype_bytes
    out_row = row if kv_bytes is None else wl.num_kv_heads * wl.head_size * kv_bytes
    return (wl.num_seqs if num_seqs is None else num_seqs) * 2 * (row + out_row)


def load_traffic(kernel_hash: str, unfused: bool, path=None):
    """HBM bytes per launch of the timed decode kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source
    and workload."""
    try:
        with open(path or TRAFFIC_FILES[unfused]) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_hash:
        return None
    return t.get("bytes_per_launch")


def host_cores() -> int:
    """CPU cores this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def oracle_sample(d, max_tokens: int, seed: int = 4242):
    """A seeded subset of the batch's sequences for the CPU oracle: sequences
    in a seeded random order until their context tokens reach max_tokens
    (at least one sequence); all of them when the batch is that small."""
    import numpy as np
    L = d.seq_lens
    if int(L.sum()) <= max_tokens:
        return list(range(len(L)))
    picked, tot = [], 0
    for b in np.random.default_rng(seed).permutation(len(L)):
        picked.append(int(b))
        tot += int(L[b])
        if tot >= max_tokens:
            break
    return sorted(picked)


def cpu_baseline(d, min_seconds: float, fp8_scales=None, max_tokens: int = 200_000):
    """The fp64 oracle (as it stands) on this host: the decode step (write the
    new token, decode) of a seeded sample of the batch's sequences (the whole
    batch when it holds at most max_tokens context tokens), repeated until
    min_seconds of CPU time; BLAS limited to one thread, so one core is what
    it uses.  fp8_scales = (k, v): the FP8 cache step (quantise the new
    tokens, decode the codes).  Returns (seconds per pass, passes, sample)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from tests.oracle_setup import OracleSide

    wl = d.wl
    seqs = oracle_sample(d, max_tokens)
    # allocator, tables and the sample's cache (setup, untimed)
    side = OracleSide(d, seqs=seqs, fill_pool=fp8_scales is None)
    if fp8_scales is not None:
        ks, vs = fp8_scales
        side.pool = oracle.empty_pool(d.num_blocks, wl.num_kv_heads, wl.block_size,
                                      wl.head_size, np.uint8, fill=np.uint8(0x7F))
        for b in seqs:
            k, v = d.kv(b)
            oracle.reshape_and_cache(side.pool, oracle.quantize(k, ks), oracle.quantize(v, vs),
                                     side.slots_for(b, 0, int(d.seq_lens[b])))
    q = d.query()
    new_k, new_v, slots = [], [], []
    for b in seqs:
        L = int(d.seq_lens[b])
        k, v = d.kv(b)
        new_k.append(k[L - 1])
        new_v.append(v[L - 1])
        slots.append(oracle.slot_mapping(side.block_tables[b], L - 1, 1, wl.block_size)[0])
    new_k, new_v, slots = np.stack(new_k), np.stack(new_v), np.array(slots)
    reps, t0 = 0, time.perf_counter()
    with threadpool_limits(1):
        while True:
            if fp8_scales is None:
                oracle.reshape_and_cache(side.pool, new_k, new_v, slots)
                oracle.decode(q, side.pool, side.block_tables, d.seq_lens, wl.scale, seqs=seqs)
            else:
                ks, vs = fp8_scales
                oracle.reshape_and_cache(side.pool, oracle.quantize(new_k, ks),
                                         oracle.quantize(new_v, vs), slots)
                oracle.decode(q, side.pool, side.block_tables, d.seq_lens, wl.scale, seqs=seqs,
                              k_scale=ks, v_scale=vs)
            reps += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
    dt = (time.perf_counter() - t0) / reps
    return dt, reps, seqs


def host_step_us(d, partition_size: int, steps: int = 200, native: bool = True) -> float:
    """Host metadata of one decode step, updated incrementally as the engine's
    CPU side does it between steps: every running sequence gains one token;
    a sequence whose new token starts a block takes one block from the
    free_block_queue (libpa allocator) into its table row; the new tokens'
    slots and the work plan are rebuilt.  native: one pa_decode_step_prepare
    call per step; otherwise the same step composed in Python from the
    allocator, slot-mapping and plan calls.  Average over `steps`
    consecutive steps, in microseconds (the uploads of the changed rows are
    not included)."""
    import numpy as np
    from paged_attention_kv_block_amd import host, ops
    bs = d.wl.block_size
    L = np.ascontiguousarray(d.seq_lens, dtype=np.int32).copy()
    width = int(max(-(-int(x) // bs) for x in L)) + steps // bs + 2
    extra = int(sum(-(-(int(x) + steps) // bs) - -(-int(x) // bs) for x in L))
    alloc = ops.Allocator(max(d.num_blocks, int(sum(-(-int(x) // bs) for x in L)) + extra),
                          None)
    bt = host.decode_block_tables(alloc, L, bs, width)
    msl = int(L.max()) + steps
    slots = np.zeros(L.size, np.int64)
    parts = 1 if partition_size <= 0 else -(-msl // partition_size)
    plan = np.zeros(L.size * parts, np.int32)
    t0 = time.perf_counter()
    if native:
        st = ops.DecodeStep(alloc, bt, L, bs, msl, partition_size)
        t0 = time.perf_counter()
        for _ in range(steps):
            st.prepare()
    else:
        for _ in range(steps):
            cross = np.flatnonzero(L % bs == 0)       # the new token opens a block
            if cross.size:
                bt[cross, L[cross] // bs] = alloc.allocate(int(cross.size))
            ops.slot_mapping(bt, L, 1, bs)
            L += 1
            ops.decode_plan(L, msl, partition_size)
    return (time.perf_counter() - t0) * 1e6 / steps


def prefill_flops(seq_lens, chunk_lens, num_q_heads: int, head_size: int) -> int:
    """Algorithmic flops of the causal chunks: query i of a chunk of C sits at
    position L - C + i and sees L - C + i + 1 keys; 2 flops of q.k and 2 of
    p.v per (query head, visible key, dim)."""
    pairs = 0
    for L, C in zip(seq_lens, chunk_lens):
        L, C = int(L), int(C)
        pairs += C * (L - C) + C * (C + 1) // 2
    return 4 * head_size * num_q_heads * pairs


def cpu_baseline_prefill(d, min_seconds: float):
    """The fp64 oracle on this host: whole sequences of the chunked-prefill
    step (write the chunk's keys/values, attend) until min_seconds; returns
    (seconds, flops done, sequences done)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from tests.oracle_setup import OracleSide

    wl = d.wl
    side = OracleSide(d)
    qsl = side.query_start_loc()
    chunks = wl.chunk_lens()
    done, flops, t0 = 0, 0, time.perf_counter()
    with threadpool_limits(1):
        while True:
            b = done % wl.num_seqs
            L, C = int(d.seq_lens[b]), int(chunks[b])
            k, v = d.kv(b)
            slots = oracle.slot_mapping(side.block_tables[b], L - C, C, wl.block_size)
            oracle.reshape_and_cache(side.pool, k[L - C:], v[L - C:], slots)
            oracle.prefill_chunk(d.query(), qsl, side.pool, side.block_tables, d.seq_lens,
                                 wl.scale, seqs=[b])
            flops += prefill_flops([L], [C], wl.num_q_heads, wl.head_size)
            done += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
    return time.perf_counter() - t0, flops, done


def bench_prefill(a, d, dev):
    """Chunked prefill with a shared prefix: pa_reshape_and_cache of every
    chunk token, then pa_prefill_chunk; MFMA roofline of the prefill kernel."""
    import numpy as np
    import torch
    from paged_attention_kv_block_amd import host, ops

    wl = d.wl
    B, Hq, Hkv, D, bs = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_size, wl.block_size
    seq_lens = d.seq_lens
    chunks = np.asarray(wl.chunk_lens(), dtype=np.int64)
    msl = int(seq_lens.max())

    def dev_tensor(arr):
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)

    ops.lib()   # load the library first: the timer covers the metadata only
    t0 = time.perf_counter()
    alloc = ops.Allocator(d.num_blocks, d.pool_order)
    own = int(seq_lens[0]) - wl.prefix_tokens
    bt = host.prefill_block_tables(alloc, B, wl.prefix_tokens, own, bs, True)
    chunk_slots = np.concatenate([ops.slot_mapping(bt[b], int(seq_lens[b]) - int(chunks[b]),
                                                   int(chunks[b]), bs) for b in range(B)])
    qsl = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    host_us = (time.perf_counter() - t0) * 1e6

    # cache holds every token before the chunks (the shared prefix once)
    pool0 = torch.zeros((d.num_blocks, 2, Hkv, bs, D), dtype=torch.bfloat16, device=dev)
    ks, vs, sl, cks, cvs = [], [], [], [], []
    for b in range(B):
        L, C = int(seq_lens[b]), int(chunks[b])
        k, v = d.kv(b)
        lo = 0 if b == 0 else wl.prefix_tokens
        ks.append(k[lo:L - C])
        vs.append(v[lo:L - C])
        sl.append(ops.slot_mapping(bt[b], lo, L - C - lo, bs))
        cks.append(k[L - C:])
        cvs.append(v[L - C:])
    ops.reshape_and_cache(dev_tensor(np.concatenate(ks)), dev_tensor(np.concatenate(vs)),
                          torch.from_numpy(np.concatenate(sl)).to(dev), pool0)
    del ks, vs
    pool_bytes = pool0.numel() * pool0.element_size()
    R = max(1, -(-a.rotate_mb * (1 << 20) // pool_bytes))
    pools = [pool0] + [pool0.clone() for _ in range(R - 1)]
    ck, cv = dev_tensor(np.concatenate(cks)), dev_tensor(np.concatenate(cvs))
    slots_dev = torch.from_numpy(chunk_slots).to(dev)
    q = dev_tensor(d.query())
    out = torch.empty_like(q)
    qsl_dev = torch.from_numpy(qsl).to(dev)
    bt_dev = torch.from_numpy(bt).to(dev)
    sl_dev = torch.from_numpy(np.ascontiguousarray(seq_lens, dtype=np.int32)).to(dev)
    max_q = int(chunks.max())
    scale = float(wl.scale)
    torch.cuda.synchronize()

    def step(pool):
        ops.reshape_and_cache(ck, cv, slots_dev, pool)
        ops.prefill_chunk(out, q, qsl_dev, max_q, pool, bt_dev, sl_dev, msl, scale)

    def prefill_only(pool):
        ops.prefill_chunk(out, q, qsl_dev, max_q, pool, bt_dev, sl_dev, msl, scale)

    def capture(fn, n):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(min(n, R)):
                fn(pools[i % R])
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(pools[i % R])
        return g

    g_warm = capture(step, max(1, a.warmup))
    g_step = capture(step, a.steps)
    g_pf = capture(prefill_only, a.steps)
    g_warm.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g_step.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / a.steps
    g_pf.replay()
    torch.cuda.synchronize()
    e0.record()
    g_pf.replay()
    e1.record()
    torch.cuda.synchronize()
    pf_us = e0.elapsed_time(e1) * 1e3 / a.steps

    flops = prefill_flops(seq_lens, chunks, Hq, D)
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (pf_us * 1e-6) / 1e12
    res = {
        "metric": "paged-attn prefill-chunk TFLOP/s (causal, algorithmic), 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) keys/values/queries; no weights)",
        "config": {
            "workload": wl.name, "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_size": D, "block_size": bs, "chunk_tokens": int(chunks.sum()),
            "shared_prefix_tokens": wl.prefix_tokens, "max_seq_len": msl,
            "pool_blocks": d.num_blocks, "pool_copies_rotated": R, "parallelism": "none (1 GPU)",
        },
        "host_metadata_us": round(host_us, 1),
        "roofline": {
            "kernel": "pa_prefill_chunk (prefill_wide_kernel)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": load_traffic(source_hash(PREFILL_SOURCES), False, PREFILL_TRAFFIC),
            "algorithmic_flops_per_launch": flops,
            "avg_launch_us": round(pf_us, 3),
        },
    }
    if not a.no_cpu_baseline:
        dt, cflops, nseq = cpu_baseline_prefill(d, a.cpu_seconds)
        res["cpu_baseline"] = {
            "value": round(cflops / dt / 1e12, 8),
            "unit": "TFLOP/s",
            "cores": 1,
            "host_cores": host_cores(),
            "blas_threads": 1,
            "kind": "oracle",
            "sample": f"{nseq} of the {B} sequences of the {wl.name} step (write the chunk's "
                      f"keys/values, attend), fp64 numpy, BLAS 1 thread; {dt:.1f} s",
        }
    print(json.dumps(res), flush=True)
    return 0


def varlen_bytes(wl, seq_lens, chunk_lens, kv_bytes=None) -> int:
    """Algorithmic bytes of one pa_attention_varlen launch: every context
    token's K/V once, query rows in, output rows out, the used block-table
    entries, seq_lens and query_start_loc.  kv_bytes as decode_bytes."""
    db = wl.dtype_bytes
    kb = db if kv_bytes is None else kv_bytes
    kv = int(sum(int(L) for L in seq_lens)) * 2 * wl.num_kv_heads * wl.head_size * kb
    rows = int(sum(int(C) for C in chunk_lens))
    qo = 2 * rows * wl.num_q_heads * wl.head_size * db
    bt = sum((int(L) + wl.block_size - 1) // wl.block_size for L in seq_lens) * 4
    return kv + qo + bt + 4 * (2 * len(seq_lens) + 1)


def cpu_baseline_mixed(d, min_seconds: float):
    """The fp64 oracle on this host over a bounded sample of the mixed step:
    sequences in turn (write the step's new keys/values, attend with the
    chunked-prefill definition, which covers the one-row decode sequences),
    until min_seconds; returns (seconds, algorithmic bytes, sequences)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from tests.oracle_setup import OracleSide

    wl = d.wl
    chunks = wl.chunk_lens()
    npre = sum(1 for c in chunks if c != chunks[-1])   # the decode sequences come last
    # alternate chunk sequences and decode rows so the sample has both kinds
    order = []
    for i in range(wl.num_seqs):
        order.append(i % npre if i % 2 == 0 else npre + (i // 2) % (wl.num_seqs - npre))
    order = order[:16]
    side = OracleSide(d, seqs=sorted(set(order)))
    qsl = side.query_start_loc()
    q = d.query()
    done, nbytes, t0 = 0, 0, time.perf_counter()
    with threadpool_limits(1):
        while True:
            b = order[done % len(order)]
            L, C = int(d.seq_lens[b]), int(chunks[b])
            k, v = d.kv(b)
            slots = oracle.slot_mapping(side.block_tables[b], L - C, C, wl.block_size)
            oracle.reshape_and_cache(side.pool, k[L - C:], v[L - C:], slots)
            oracle.prefill_chunk(q, qsl, side.pool, side.block_tables, d.seq_lens, wl.scale,
                                 seqs=[b])
            nbytes += varlen_bytes(wl, [L], [C])
            done += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
    return time.perf_counter() - t0, nbytes, done


def bench_mixed(a, dev):
    """One continuous-batching step over a flattened batch: 16 prefill chunks
    of 256 rows after 2560 cached tokens and 240 decode rows of log-normal
    length (Llama-3-8B-shaped heads).  The step writes the new tokens'
    keys/values (pa_reshape_and_cache) and runs pa_attention_varlen, one
    launch for both kinds of rows; the same step with pa_prefill_chunk and
    pa_decode as two launches is timed beside it.  With --spec-rows C every
    decode sequence has C rows (a speculative step): the varlen launch runs
    them as multi-row decode items, and the second of the two launches is
    pa_decode_multi."""
    import numpy as np
    import torch
    from paged_attention_kv_block_amd import host, inputs, ops

    Cd = max(1, int(a.spec_rows))          # rows per decode sequence
    d = inputs.mixed_step(decode_rows=Cd)
    wl = d.wl
    B, Hq, Hkv, D, bs = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_size, wl.block_size
    seq_lens = d.seq_lens
    chunks = np.asarray(wl.chunk_lens(), dtype=np.int64)
    npre = int(np.sum(chunks != Cd))        # the chunk sequences come first
    assert np.all(chunks[:npre] > Cd) and np.all(chunks[npre:] == Cd)
    msl = int(seq_lens.max())
    P = 512 if a.partition_size is None else a.partition_size

    def dev_tensor(arr):
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)

    ops.lib()   # load the library first: the timer covers the metadata only
    t0 = time.perf_counter()
    alloc = ops.Allocator(d.num_blocks, d.pool_order)
    bt = host.decode_block_tables(alloc, seq_lens, bs)
    qsl = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    new_slots = np.concatenate([ops.slot_mapping(bt[b], int(seq_lens[b]) - int(chunks[b]),
                                                 int(chunks[b]), bs) for b in range(B)])
    vplan, vnpre = ops.varlen_plan(qsl, seq_lens, msl, Hq, Hkv, P)
    host_us = (time.perf_counter() - t0) * 1e6
    dplan = ops.decode_plan(seq_lens[npre:], msl, P)

    # the cache holds every token before the step; the step writes the rest
    pool = torch.zeros((d.num_blocks, 2, Hkv, bs, D), dtype=torch.bfloat16, device=dev)
    ks, vs, sl, nks, nvs = [], [], [], [], []
    for b in range(B):
        L, C = int(seq_lens[b]), int(chunks[b])
        k, v = d.kv(b)
        ks.append(k[:L - C])
        vs.append(v[:L - C])
        sl.append(ops.slot_mapping(bt[b], 0, L - C, bs))
        nks.append(k[L - C:])
        nvs.append(v[L - C:])
    ops.reshape_and_cache(dev_tensor(np.concatenate(ks)), dev_tensor(np.concatenate(vs)),
                          torch.from_numpy(np.concatenate(sl)).to(dev), pool)
    del ks, vs
    nk, nv = dev_tensor(np.concatenate(nks)), dev_tensor(np.concatenate(nvs))
    slots_dev = torch.from_numpy(new_slots).to(dev)
    q = dev_tensor(d.query())
    T = q.shape[0]
    Tpre = int(qsl[npre])
    out = torch.empty_like(q)
    qsl_dev = torch.from_numpy(qsl).to(dev)
    qsl_pre = qsl_dev[:npre + 1]
    bt_dev = torch.from_numpy(bt).to(dev)
    sl_dev = torch.from_numpy(np.ascontiguousarray(seq_lens, dtype=np.int32)).to(dev)
    vplan_dev = torch.from_numpy(vplan).to(dev)
    dplan_dev = torch.from_numpy(dplan).to(dev)
    ws = ops.decode_workspace(B, Hq, Hkv, D, msl, P, dev)
    ws_dec = (ops.decode_workspace(B - npre, Hq, Hkv, D, msl, P, dev) if Cd == 1 else
              ops.decode_multi_workspace(B - npre, Cd, Hq, Hkv, D, msl, P, dev))
    scale = float(wl.scale)
    msl_pre = int(seq_lens[:npre].max())
    max_q = int(chunks[:npre].max())
    torch.cuda.synchronize()

    def varlen():
        ops.attention_varlen(out, q, qsl_dev, pool, bt_dev, sl_dev, msl, scale, vplan_dev, P, ws)

    def separate():
        ops.prefill_chunk(out[:Tpre], q[:Tpre], qsl_pre, max_q, pool, bt_dev[:npre],
                          sl_dev[:npre], msl_pre, scale)
        if Cd == 1:
            ops.decode(out[Tpre:], q[Tpre:], pool, bt_dev[npre:], sl_dev[npre:], msl, scale, P,
                       ws_dec, plan=dplan_dev)
        else:
            ops.decode_multi(out[Tpre:], q[Tpre:], pool, bt_dev[npre:], sl_dev[npre:], msl,
                             scale, Cd, P, ws_dec, plan=dplan_dev)

    def step():
        ops.reshape_and_cache(nk, nv, slots_dev, pool)
        varlen()

    def step_separate():
        ops.reshape_and_cache(nk, nv, slots_dev, pool)
        separate()

    def capture(fn, n):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        return g

    def timed(g, n):
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n   # microseconds per step

    g_warm = capture(step, max(1, a.warmup))
    g_warm.replay()
    torch.cuda.synchronize()
    step_us = timed(capture(step, a.steps), a.steps)
    sep_us = timed(capture(step_separate, a.steps), a.steps)
    var_us = timed(capture(varlen, a.steps), a.steps)
    two_us = timed(capture(separate, a.steps), a.steps)

    kbytes = varlen_bytes(wl, seq_lens, chunks)
    wbytes = 2 * 2 * int(chunks.sum()) * Hkv * D * 2        # read + write the new K and V rows
    flops = prefill_flops(seq_lens, chunks, Hq, D)
    value = (kbytes + wbytes) / (step_us * 1e-6) / 1e9
    achieved = kbytes / (var_us * 1e-6) / 1e9
    res = {
        "metric": "paged-attn varlen step GB/s (decode rows + prefill chunks, one launch), 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(step_us * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) keys/values/queries; no weights)",
        "config": {
            "workload": "mixed-step-llama3-8b" + (f"-spec{Cd}" if Cd > 1 else ""),
            "sequences": B, "prefill_chunks": npre,
            "chunk_tokens": int(chunks[:npre].sum()), "decode_sequences": B - npre,
            "rows_per_decode_sequence": Cd,
            "num_q_heads": Hq, "num_kv_heads": Hkv, "head_size": D, "block_size": bs,
            "context_tokens": int(seq_lens.sum()), "max_seq_len": msl, "partition_size": P,
            "pool_blocks": d.num_blocks, "parallelism": "none (1 GPU)",
        },
        "host_metadata_us": round(host_us, 1),
        "step_us_one_launch": round(step_us, 2),
        "step_us_two_launches": round(sep_us, 2),
        "attention_us_one_launch": round(var_us, 2),
        "attention_us_two_launches": round(two_us, 2),
        "attention_tflops": round(flops / (var_us * 1e-6) / 1e12, 2),
        "roofline": {
            "kernel": "pa_attention_varlen (varlen_kernel)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (load_traffic(source_hash(VARLEN_SOURCES), False, VARLEN_TRAFFIC)
                        if P == 512 and Cd == 1 else None),
            "algorithmic_bytes_per_launch": kbytes,
            "algorithmic_flops_per_launch": flops,
            "mfma_frac": round(flops / (var_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "avg_launch_us": round(var_us, 3),
        },
    }
    if not a.no_cpu_baseline:
        dt, cbytes, nseq = cpu_baseline_mixed(d, a.cpu_seconds)
        res["cpu_baseline"] = {
            "value": round(cbytes / dt / 1e9, 6),
            "unit": "GB/s",
            "cores": 1,
            "host_cores": host_cores(),
            "blas_threads": 1,
            "kind": "oracle",
            "sample": f"{nseq} sequences of the mixed step, chunk sequences and decode rows "
                      f"alternating (write the step's keys/values, attend), fp64 numpy, BLAS "
                      f"1 thread; {dt:.1f} s",
        }
    print(json.dumps(res), flush=True)
    return 0


def cpu_baseline_spec(d, min_seconds: float, fp8_scales=None):
    """The fp64 oracle on this host over a bounded sample of a speculative
    step: sequences spread over the batch in turn, each one's C rows as the
    chunked-prefill definition gives them (its cache filled beforehand,
    quantised to FP8 codes with fp8_scales = (k, v) when given), until
    min_seconds; returns (seconds, algorithmic bytes, sequences)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from tests.oracle_setup import OracleSide

    wl = d.wl
    B = wl.num_seqs
    sample = sorted(set(int(x) for x in np.linspace(0, B - 1, min(B, 8))))
    side = OracleSide(d, seqs=sample)
    ks = vs = 1.0
    kvb = None
    if fp8_scales is not None:
        ks, vs = fp8_scales
        kvb = 1
        side.pool = np.stack([oracle.quantize(side.pool[:, 0], ks),
                              oracle.quantize(side.pool[:, 1], vs)], axis=1)
    qsl = side.query_start_loc()
    q = d.query()
    chunks = wl.chunk_lens()
    done, nbytes, t0 = 0, 0, time.perf_counter()
    with threadpool_limits(1):
        while True:
            b = sample[done % len(sample)]
            oracle.prefill_chunk(q, qsl, side.pool, side.block_tables, d.seq_lens, wl.scale,
                                 seqs=[b], k_scale=ks, v_scale=vs)
            nbytes += varlen_bytes(wl, [int(d.seq_lens[b])], [int(chunks[b])], kvb)
            done += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
    return time.perf_counter() - t0, nbytes, done


def bench_prefix_cache(a, dev):
    """Prefix caching on the shared-prefix workload: 16 requests, each a
    2816-token prompt made of a common 2048-token prefix and 768 tokens of
    its own (32/8 heads, D 128, bf16).  Host: libpa's allocator with its
    prefix cache serves the requests in turn (lookup of all but the last
    token, allocation of the rest, registration of the full blocks), timed
    per request.  Device: the prefill of the 16 prompts without the cache
    (every request computes all its 2816 tokens over its own blocks) against
    the same with it (the first request computes everything, the others only
    their 768 tokens over the cached prefix blocks), each as one
    pa_prefill_chunk launch; the rows both compute must agree."""
    import numpy as np
    import torch
    from paged_attention_kv_block_amd import host, inputs, ops

    d = inputs.draw(3)
    wl = d.wl
    B, Hq, Hkv, D, bs = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_size, wl.block_size
    L = int(d.seq_lens[0])
    pre = wl.prefix_tokens
    nblk = -(-L // bs)
    rng = np.random.default_rng(3003)
    shared = rng.integers(0, 32000, size=pre)
    tokens = [np.concatenate([shared, rng.integers(0, 32000, size=L - pre)]).astype(np.int32)
              for _ in range(B)]
    q_all = inputs.round_to_bf16_bits(
        rng.standard_normal(size=(B, L, Hq, D), dtype=np.float32))   # every prompt position

    def dev_tensor(arr):
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)

    # host: the prefix cache serves the requests in turn
    ops.lib()
    alloc = ops.Allocator(d.num_blocks, d.pool_order)
    alloc.enable_prefix_cache(bs)
    bt_c = np.full((B, nblk), -1, dtype=np.int32)
    starts = []
    t0 = time.perf_counter()
    for b in range(B):
        hits = alloc.acquire_prefix(tokens[b][:-1])
        row = hits + alloc.allocate(nblk - len(hits))
        alloc.insert_prefix(tokens[b], row)
        bt_c[b] = row
        starts.append(len(hits) * bs)
    host_us = (time.perf_counter() - t0) * 1e6 / B
    _, (cached_blocks, hit_blocks, evictions) = alloc.export_prefix_cache()

    # without the cache: every request has its own blocks for all its tokens
    n_u = int(np.ceil(1.1 * B * nblk))
    alloc_u = ops.Allocator(n_u, np.random.default_rng(3004).permutation(n_u).astype(np.int32))
    bt_u = host.decode_block_tables(alloc_u, [L] * B, bs)

    def fill(pool, bt, first):
        for b in range(B):
            k, v = d.kv(b)
            sl = ops.slot_mapping(bt[b], first[b], L - first[b], bs)
            ops.reshape_and_cache(dev_tensor(k[first[b]:]), dev_tensor(v[first[b]:]),
                                  torch.from_numpy(sl).to(dev), pool)

    pool_c = torch.zeros((d.num_blocks, 2, Hkv, bs, D), dtype=torch.bfloat16, device=dev)
    pool_u = torch.zeros((n_u, 2, Hkv, bs, D), dtype=torch.bfloat16, device=dev)
    fill(pool_c, bt_c, starts)          # each request writes the tokens it computes
    fill(pool_u, bt_u, [0] * B)
    rows_c = [L - s0 for s0 in starts]
    q_c = dev_tensor(np.concatenate([q_all[b, starts[b]:] for b in range(B)]))
    q_u = dev_tensor(q_all.reshape(B * L, Hq, D))
    out_c, out_u = torch.empty_like(q_c), torch.empty_like(q_u)
    qsl_c = torch.from_numpy(np.concatenate([[0], np.cumsum(rows_c)]).astype(np.int32)).to(dev)
    qsl_u = torch.from_numpy(np.arange(0, B * L + 1, L, dtype=np.int32)).to(dev)
    sl_dev = torch.full((B,), L, dtype=torch.int32, device=dev)
    btc_dev, btu_dev = torch.from_numpy(bt_c).to(dev), torch.from_numpy(bt_u).to(dev)
    scale = float(wl.scale)
    torch.cuda.synchronize()

    def cached():
        ops.prefill_chunk(out_c, q_c, qsl_c, max(rows_c), pool_c, btc_dev, sl_dev, L, scale)

    def uncached():
        ops.prefill_chunk(out_u, q_u, qsl_u, L, pool_u, btu_dev, sl_dev, L, scale)

    def timed(fn, n):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    n = max(5, a.steps // 10)
    c_us = timed(cached, n)
    u_us = timed(uncached, n)
    # the rows both launches compute (positions >= the cached prefix) agree
    diff, exact = 0.0, True
    off = 0
    for b in range(B):
        oc = out_c[off:off + rows_c[b]].float()
        ou = out_u[b * L + starts[b]:(b + 1) * L].float()
        diff = max(diff, float((oc - ou).abs().max()))
        exact = exact and torch.equal(out_c[off:off + rows_c[b]].view(torch.int16),
                                      out_u[b * L + starts[b]:(b + 1) * L].view(torch.int16))
        off += rows_c[b]
    assert diff <= 2e-2, diff
    f_c = prefill_flops([L] * B, rows_c, Hq, D)
    f_u = prefill_flops([L] * B, [L] * B, Hq, D)
    achieved = f_c / (c_us * 1e-6) / 1e12
    res = {
        "metric": "prefix-cache prefill: prompt tokens served per second, 16 requests sharing a "
                  "2048-token prefix, 1 GPU",
        "value": round(B * L / (c_us * 1e-6), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": 1,
        "ms_per_step": round(c_us * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) keys/values/queries, random token ids; no weights)",
        "config": {
            "workload": "prefix-cache-shared-prefix-b16", "requests": B, "prompt_tokens": L,
            "shared_prefix_tokens": pre, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_size": D, "block_size": bs, "parallelism": "none (1 GPU)",
        },
        "host_us_per_request": round(host_us, 1),
        "prefix_cache": {"hit_blocks": hit_blocks, "cached_blocks": cached_blocks,
                         "evictions": evictions, "computed_tokens": int(sum(rows_c)),
                         "computed_tokens_without_cache": B * L},
        "prefill_us_with_cache": round(c_us, 2),
        "prefill_us_without_cache": round(u_us, 2),
        "speedup": round(u_us / c_us, 3),
        "shared_rows_max_abs_diff": diff,
        "shared_rows_bit_identical": bool(exact),
        "roofline": {
            "kernel": "pa_prefill_chunk (prefill_wide_kernel), with the cache",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
            "algorithmic_flops_per_launch": f_c,
            "algorithmic_flops_without_cache": f_u,
            "avg_launch_us": round(c_us, 3),
        },
    }
    if not a.no_cpu_baseline:
        dt, cflops, nseq = cpu_baseline_prefill(d, a.cpu_seconds)
        res["cpu_baseline"] = {
            "value": round(cflops / dt / 1e12, 8),
            "unit": "TFLOP/s",
            "cores": 1,
            "host_cores": host_cores(),
            "blas_threads": 1,
            "kind": "oracle",
            "sample": f"{nseq} sequences of the shared-prefix chunked-prefill step (the same "
                      f"attention definition, 256-row chunks over the cached prefix), fp64 "
                      f"numpy, BLAS 1 thread; {dt:.1f} s",
        }
    print(json.dumps(res), flush=True)
    return 0


def bench_spec(a, dev):
    """A speculative-decoding verification step: every sequence of a decode
    batch checks C = --spec-rows tokens at once (C - 1 draft tokens and the
    one after them), i.e. a causal chunk of C query rows at the end of its
    context.  The batch, heads and lengths are those of decode workload
    --workload (lengths include the C new tokens).  The timed launch is
    pa_decode_multi (the decode kernel with (row, head) matrix columns,
    split-K as the workload's decode); beside it, on the same cache,
    pa_attention_varlen and pa_prefill_chunk (the same rows as 128-row
    query tiles) and, for scale, pa_decode with one row per sequence.
    With --kv-cache fp8 the cache holds E4M3 codes (per-tensor scales) and
    the timed launch is pa_decode_multi_fp8, beside pa_decode_fp8 with one
    row per sequence."""
    import numpy as np
    import torch
    from paged_attention_kv_block_amd import host, inputs, ops

    base = inputs.workload(a.workload)
    if base.kind != "decode" or base.dtype != "bf16":
        print("bench.py: --spec-rows needs a bf16 decode workload (1, 2 or 4)", file=sys.stderr)
        return 2
    C = int(a.spec_rows)
    fp8 = a.kv_cache == "fp8"
    d0 = inputs.draw(a.workload)
    B, Hq, Hkv, D, bs = base.num_seqs, base.num_q_heads, base.num_kv_heads, base.head_size, \
        base.block_size
    seq_lens = np.maximum(d0.seq_lens, C).astype(np.int32)
    chunks = np.full(B, C, dtype=np.int64)
    d = inputs.custom(f"spec-verify-{base.name}", kind="prefill", seq_lens=seq_lens,
                      chunk_lens=chunks.tolist(), num_q_heads=Hq, num_kv_heads=Hkv,
                      head_size=D, seed=3000 + a.workload, index=200 + a.workload)
    msl = int(seq_lens.max())
    P = default_partition(base) if a.partition_size is None else a.partition_size

    def dev_tensor(arr):
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)

    alloc = ops.Allocator(d.num_blocks, d.pool_order)
    bt = host.decode_block_tables(alloc, seq_lens, bs)
    qsl = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    ops.lib()   # load the library first: the timer covers the metadata only
    t0 = time.perf_counter()
    vplan, _ = ops.varlen_plan(qsl, seq_lens, msl, Hq, Hkv, P)
    host_us = (time.perf_counter() - t0) * 1e6
    dplan = ops.decode_plan(seq_lens, msl, P)
    k_scale = v_scale = 1.0
    if fp8:   # per-tensor scales mapping the largest |key| / |value| to 448
        kmax = vmax = 0.0
        for b in range(B):
            k, v = d.kv(b)
            kmax = max(kmax, float(np.max(np.abs((k.astype(np.uint32) << 16).view(np.float32)))))
            vmax = max(vmax, float(np.max(np.abs((v.astype(np.uint32) << 16).view(np.float32)))))
        k_scale, v_scale = max(kmax, 1e-3) / 448.0, max(vmax, 1e-3) / 448.0
    pool0 = torch.zeros((d.num_blocks, 2, Hkv, bs, D),
                        dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
    for lo in range(0, B, 32):           # fill in slices to bound host memory
        ks, vs, sl = [], [], []
        for b in range(lo, min(B, lo + 32)):
            k, v = d.kv(b)
            ks.append(k)
            vs.append(v)
            sl.append(ops.slot_mapping(bt[b], 0, int(seq_lens[b]), bs))
        kd, vd = dev_tensor(np.concatenate(ks)), dev_tensor(np.concatenate(vs))
        sld = torch.from_numpy(np.concatenate(sl)).to(dev)
        if fp8:
            ops.reshape_and_cache_fp8(kd, vd, sld, pool0, k_scale, v_scale)
        else:
            ops.reshape_and_cache(kd, vd, sld, pool0)
        del ks, vs, kd, vd
    pool_bytes = pool0.numel() * pool0.element_size()
    R = max(1, -(-a.rotate_mb * (1 << 20) // pool_bytes))
    pools = [pool0] + [pool0.clone() for _ in range(R - 1)]
    q = dev_tensor(d.query())
    out = torch.empty_like(q)
    q1 = q.view(B, C, Hq, D)[:, C - 1].contiguous()
    out1 = torch.empty_like(q1)
    qsl_dev = torch.from_numpy(qsl).to(dev)
    bt_dev = torch.from_numpy(bt).to(dev)
    sl_dev = torch.from_numpy(seq_lens).to(dev)
    vplan_dev = torch.from_numpy(vplan).to(dev)
    dplan_dev = torch.from_numpy(dplan).to(dev)
    ws = ops.decode_workspace(B, Hq, Hkv, D, msl, P, dev)
    ws_multi = ops.decode_multi_workspace(B, C, Hq, Hkv, D, msl, P, dev)
    scale = float(base.scale)
    torch.cuda.synchronize()

    def multi(pool):
        if fp8:
            ops.decode_multi_fp8(out, q, pool, bt_dev, sl_dev, msl, scale, k_scale, v_scale, C, P,
                                 ws_multi, plan=dplan_dev)
        else:
            ops.decode_multi(out, q, pool, bt_dev, sl_dev, msl, scale, C, P, ws_multi,
                             plan=dplan_dev)

    def varlen(pool):
        ops.attention_varlen(out, q, qsl_dev, pool, bt_dev, sl_dev, msl, scale, vplan_dev, P, ws)

    def prefill(pool):
        ops.prefill_chunk(out, q, qsl_dev, C, pool, bt_dev, sl_dev, msl, scale)

    def decode1(pool):
        if fp8:
            ops.decode_fp8(out1, q1, pool, bt_dev, sl_dev, msl, scale, k_scale, v_scale, P, ws,
                           plan=dplan_dev)
        else:
            ops.decode(out1, q1, pool, bt_dev, sl_dev, msl, scale, P, ws, plan=dplan_dev)

    def timed(fn, n):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(min(n, R)):
                fn(pools[i % R])
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(pools[i % R])
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    multi_us = timed(multi, a.steps)
    var_us = None if fp8 else timed(varlen, a.steps)      # no FP8 variant of these two
    pre_us = None if fp8 else timed(prefill, a.steps)
    dec_us = timed(decode1, a.steps)
    kbytes = varlen_bytes(d.wl, seq_lens, chunks, 1 if fp8 else None)
    flops = prefill_flops(seq_lens, chunks, Hq, D)
    achieved = kbytes / (multi_us * 1e-6) / 1e9
    res = {
        "metric": "paged-attn speculative-verify step GB/s (C query rows per sequence), 1 GPU",
        "value": round(achieved, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(multi_us * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) keys/values/queries; no weights)",
        "config": {
            "workload": f"spec-verify-{base.name}", "batch": B, "rows_per_sequence": C,
            "num_q_heads": Hq, "num_kv_heads": Hkv, "head_size": D, "block_size": bs,
            "context_tokens": int(seq_lens.sum()), "max_seq_len": msl, "partition_size": P,
            "pool_blocks": d.num_blocks, "pool_copies_rotated": R,
            "kv_cache": ("fp8-e4m3, per-tensor scales k %.6g v %.6g" % (k_scale, v_scale)
                         if fp8 else "bf16"),
            "parallelism": "none (1 GPU)",
        },
        "host_plan_us": round(host_us, 1),
        "attention_us_decode_multi": round(multi_us, 2),
        "attention_us_varlen": None if var_us is None else round(var_us, 2),
        "attention_us_prefill_chunk": None if pre_us is None else round(pre_us, 2),
        "decode_us_one_row": round(dec_us, 2),
        "roofline": {
            "kernel": ("pa_decode_multi_fp8 (decode_kernel, multi-row, FP8 cache)" if fp8
                       else "pa_decode_multi (decode_kernel, multi-row)"),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (load_traffic(source_hash(DECODE_SOURCES), False,
                                     MULTI_FP8_TRAFFIC if fp8 else MULTI_TRAFFIC)
                        if a.workload == 2 and C == 4 and P == 512 else None),
            "algorithmic_bytes_per_launch": kbytes,
            "algorithmic_flops_per_launch": flops,
            "avg_launch_us": round(multi_us, 3),
        },
    }
    if not a.no_cpu_baseline:
        dt, cbytes, nseq = cpu_baseline_spec(d, a.cpu_seconds,
                                             (k_scale, v_scale) if fp8 else None)
        res["cpu_baseline"] = {
            "value": round(cbytes / dt / 1e9, 6),
            "unit": "GB/s",
            "cores": 1,
            "host_cores": host_cores(),
            "blas_threads": 1,
            "kind": "oracle",
            "sample": f"{nseq} sequences of the step in turn (up to 8 spread over the batch, "
                      f"their {C} rows each), fp64 numpy, BLAS 1 thread; {dt:.1f} s",
        }
    print(json.dumps(res), flush=True)
    return 0


def bench_graphs(a, dev):
    """Decode steps replayed from the graphs captured per warm-up batch size
    (pa_decode_graphs_*), at several batch sizes B up to the workload's:
    each replay takes the smallest captured size that fits and pads the
    rest with seq_len 0.  --layers L stacks L layers (each its own cache,
    queries and new K/V; the block tables and lengths shared), as a model's
    decode step runs attention once per layer.  Beside each: the same step
    issued eagerly (pa_decode_append per layer without a plan, as the graphs
    hold it), one ctypes call per launch.  Timed per step from the host loop
    (wall clock: what a serving loop sees) and on the device (HIP events).
    Cache copies rotate as in the decode line: one graph set per copy."""
    import numpy as np
    import torch
    from paged_attention_kv_block_amd import host, inputs, ops
    wl = inputs.workload(a.workload)
    d = inputs.draw(a.workload)
    if wl.kind != "decode" or wl.dtype != "bf16":
        print("bench.py: --graphs needs a bf16 decode workload", file=sys.stderr)
        return 2
    B, Hq, Hkv, D, bs = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_size, wl.block_size
    P = default_partition(wl) if a.partition_size is None else a.partition_size
    NL = max(1, int(a.layers))
    seq_lens = d.seq_lens
    msl = int(seq_lens.max())

    def dev_tensor(arr):
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)

    alloc = ops.Allocator(d.num_blocks, d.pool_order)
    bt = host.decode_block_tables(alloc, seq_lens, bs)
    pool0 = torch.zeros((d.num_blocks, 2, Hkv, bs, D), dtype=torch.bfloat16, device=dev)
    ks, vs, sl, new_k, new_v = [], [], [], [], []
    for b in range(B):
        L = int(seq_lens[b])
        k, v = d.kv(b)
        ks.append(k[:L - 1])
        vs.append(v[:L - 1])
        sl.append(ops.slot_mapping(bt[b], 0, L - 1, bs))
        new_k.append(k[L - 1])
        new_v.append(v[L - 1])
    ops.reshape_and_cache(dev_tensor(np.concatenate(ks)), dev_tensor(np.concatenate(vs)),
                          torch.from_numpy(np.concatenate(sl)).to(dev), pool0)
    del ks, vs
    pool_bytes = pool0.numel() * pool0.element_size()
    R = max(1, -(-a.rotate_mb * (1 << 20) // (pool_bytes * NL)))
    pools = [pool0] + [pool0.clone() for _ in range(R * NL - 1)]   # set r, layer l: r * NL + l
    q = dev_tensor(d.query()).unsqueeze(0).repeat(NL, 1, 1, 1).contiguous()
    nk = dev_tensor(np.stack(new_k)).unsqueeze(0).repeat(NL, 1, 1, 1).contiguous()
    nv = dev_tensor(np.stack(new_v)).unsqueeze(0).repeat(NL, 1, 1, 1).contiguous()
    bt_dev = torch.from_numpy(bt).to(dev)
    lens_dev = torch.from_numpy(np.ascontiguousarray(seq_lens, dtype=np.int32)).to(dev)
    sl_dev = lens_dev.clone()
    out = torch.empty_like(q)
    ws = ops.decode_workspace(B, Hq, Hkv, D, msl, P, dev)
    scale = float(wl.scale)
    sizes = sorted({1 << i for i in range(16) if (1 << i) < B} | {B})
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sets = [ops.DecodeGraphs(out, q, nk, nv, pools[r * NL:(r + 1) * NL], bt_dev, sl_dev, msl,
                                 scale, sizes, P, ws) for r in range(R)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    def timed(fn, Bx):
        for i in range(max(1, a.warmup)):
            fn(Bx, i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        h0 = time.perf_counter()
        e0.record()
        for i in range(a.steps):
            fn(Bx, i)
        e1.record()
        h1 = time.perf_counter()
        torch.cuda.synchronize()
        h2 = time.perf_counter()
        return ((h1 - h0) * 1e6 / a.steps, (h2 - h0) * 1e6 / a.steps,
                e0.elapsed_time(e1) * 1e3 / a.steps)

    def replay(Bx, i):
        sets[i % R].replay(Bx)

    def eager(Bx, i):
        r = i % R
        for layer in range(NL):
            ops.decode(out[layer, :Bx], q[layer, :Bx], pools[r * NL + layer], bt_dev[:Bx],
                       sl_dev[:Bx], msl, scale, P, ws, new_key=nk[layer, :Bx],
                       new_value=nv[layer, :Bx])

    rows = []
    for Bx in sorted({1, max(1, B // 8), max(1, B // 4) + 1, B // 2, B}):
        sl_dev.copy_(lens_dev)           # replays zero the padding lengths
        torch.cuda.synchronize()
        g_issue, g_wall, g_dev = timed(replay, Bx)
        sl_dev.copy_(lens_dev)
        torch.cuda.synchronize()
        e_issue, e_wall, e_dev = timed(eager, Bx)
        Bc = min(s for s in sizes if s >= Bx)
        step_bytes = NL * (decode_bytes(wl, seq_lens[:Bx]) + cache_write_bytes(wl, None, Bx))
        rows.append({"batch": Bx, "graph_batch": Bc,
                     "graph_step_us": round(g_dev, 2), "graph_host_issue_us": round(g_issue, 2),
                     "graph_wall_us": round(g_wall, 2),
                     "eager_step_us": round(e_dev, 2), "eager_host_issue_us": round(e_issue, 2),
                     "eager_wall_us": round(e_wall, 2),
                     "graph_gbs": round(step_bytes / (g_dev * 1e-6) / 1e9, 1),
                     "eager_gbs": round(step_bytes / (e_dev * 1e-6) / 1e9, 1)})
        log(f"graphs: B={Bx} (graph {Bc}), {NL} layer(s): replay {g_dev:.2f} us/step on the "
            f"device, {g_issue:.2f} us host issue; eager {e_dev:.2f} / {e_issue:.2f} us")
    full = rows[-1]
    for s_ in sets:
        s_.close()
    res = {
        "metric": "paged-attn decode step GB/s replayed from graphs per warm-up batch size, 1 GPU",
        "value": full["graph_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(full["graph_step_us"] * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) keys/values/queries; no weights)",
        "config": {"workload": wl.name + "-graphs", "batch": B, "layers": NL,
                   "num_q_heads": Hq, "num_kv_heads": Hkv, "head_size": D, "block_size": bs,
                   "max_seq_len": msl, "partition_size": P, "warmup_batch_sizes": sizes,
                   "cache_sets_rotated": R, "parallelism": "none (1 GPU)"},
        "by_batch": rows,
    }
    print(json.dumps(res), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=4,
                    help="workload index: decode 1, 2, 4 (0 = tiny); 3 = chunked prefill; "
                         "default 4, the long-context batch (the largest decode workload)")
    ap.add_argument("--mixed", action="store_true",
                    help="a flattened continuous-batching step: 16 prefill chunks and 240 "
                         "decode rows in one pa_attention_varlen launch")
    ap.add_argument("--prefix-cache", action="store_true",
                    help="16 requests sharing a 2048-token prefix through the allocator's "
                         "prefix cache: host cost per request and the prefill launch with "
                         "and without the cache")
    ap.add_argument("--spec-rows", type=int, default=0,
                    help="a speculative-decoding verification step: every sequence of decode "
                         "workload --workload checks this many query rows at once")
    ap.add_argument("--graphs", action="store_true",
                    help="decode workload --workload replayed from graphs captured per warm-up "
                         "batch size (pa_decode_graphs_*) at several batch sizes, beside eager "
                         "launches")
    ap.add_argument("--layers", type=int, default=1,
                    help="with --graphs: attention layers per decode step (one cache each)")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="split-K partition in tokens (default: workload's, else 256/512)")
    ap.add_argument("--rotate-mb", type=int, default=768,
                    help="total size of rotated pool copies (defeats the 256 MB Infinity Cache)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="decode step as two launches (pa_reshape_and_cache, pa_decode) "
                         "instead of pa_decode_append")
    ap.add_argument("--kv-cache", choices=["native", "fp8"], default="native",
                    help="decode workloads: keep the cache in the workload dtype (default) "
                         "or in FP8 E4M3 with per-tensor scales (pa_decode_append_fp8; with "
                         "--unfused pa_reshape_and_cache_fp8 + pa_decode_fp8; with --spec-rows "
                         "pa_decode_multi_fp8)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration)")
    a = ap.parse_args(argv)

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the library runs on one GPU only; multi-GPU sharding is not "
              "implemented (--gpus must be 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from paged_attention_kv_block_amd import host, inputs, ops

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda", 0)

    if a.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 5 copies of {n} bytes")
        return 0

    if a.mixed:
        return bench_mixed(a, dev)
    if a.prefix_cache:
        return bench_prefix_cache(a, dev)
    if a.spec_rows > 0:
        return bench_spec(a, dev)
    if a.graphs:
        return bench_graphs(a, dev)
    wl = inputs.workload(a.workload)
    d = inputs.draw(a.workload)
    if wl.kind == "prefill":
        return bench_prefill(a, d, dev)
    fp8 = a.kv_cache == "fp8"
    if fp8 and wl.dtype != "bf16":
        print("bench.py: the FP8 cache is for bf16 workloads", file=sys.stderr)
        return 2
    B, Hq, Hkv, D, bs = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_size, wl.block_size
    P = default_partition(wl) if a.partition_size is None else a.partition_size
    seq_lens = d.seq_lens
    msl = int(seq_lens.max())
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    def dev_tensor(arr):
        if wl.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)

    # ---- host metadata (engine CPU side), timed separately
    ops.lib()   # load the library first: the timer covers the metadata only
    t0 = time.perf_counter()
    alloc = ops.Allocator(d.num_blocks, d.pool_order)
    bt = host.decode_block_tables(alloc, seq_lens, bs)
    new_slots = ops.slot_mapping(bt, seq_lens - 1, 1, bs)
    plan = ops.decode_plan(seq_lens, msl, P)
    host_us = (time.perf_counter() - t0) * 1e6
    step_host_us = host_step_us(d, P)
    step_host_us_py = host_step_us(d, P, native=False)

    # ---- device inputs: cache holds tokens 0..L-2; the step writes token L-1
    pool_shape = (d.num_blocks, 2, Hkv, bs, D)
    pool0 = torch.zeros(pool_shape, dtype=torch.uint8 if fp8 else tdt, device=dev)
    ks, vs, sl = [], [], []
    new_k, new_v = [], []
    for b in range(B):
        L = int(seq_lens[b])
        k, v = d.kv(b)
        ks.append(k[:L - 1])
        vs.append(v[:L - 1])
        sl.append(ops.slot_mapping(bt[b], 0, L - 1, bs))
        new_k.append(k[L - 1])
        new_v.append(v[L - 1])
    k_scale = v_scale = 1.0
    if fp8:   # per-tensor scales mapping the largest |key| / |value| to 448
        def absmax(rows):
            return max(float(np.max(np.abs((np.asarray(x).astype(np.uint32) << 16)
                                            .view(np.float32)))) for x in rows if np.size(x))
        k_scale = absmax(ks + new_k) / 448.0
        v_scale = absmax(vs + new_v) / 448.0
        ops.reshape_and_cache_fp8(dev_tensor(np.concatenate(ks)), dev_tensor(np.concatenate(vs)),
                                  torch.from_numpy(np.concatenate(sl)).to(dev), pool0,
                                  k_scale, v_scale)
    else:
        ops.reshape_and_cache(dev_tensor(np.concatenate(ks)), dev_tensor(np.concatenate(vs)),
                              torch.from_numpy(np.concatenate(sl)).to(dev), pool0)
    del ks, vs
    pool_bytes = pool0.numel() * pool0.element_size()
    R = max(1, -(-a.rotate_mb * (1 << 20) // pool_bytes))
    pools = [pool0] + [pool0.clone() for _ in range(R - 1)]
    q = dev_tensor(d.query())
    nk, nv = dev_tensor(np.stack(new_k)), dev_tensor(np.stack(new_v))
    slots_dev = torch.from_numpy(new_slots).to(dev)
    plan_dev = torch.from_numpy(plan).to(dev)
    bt_dev = torch.from_numpy(bt).to(dev)
    sl_dev = torch.from_numpy(np.ascontiguousarray(seq_lens, dtype=np.int32)).to(dev)
    out = torch.empty_like(q)
    ws = ops.decode_workspace(B, Hq, Hkv, D, msl, P, dev)
    scale = float(wl.scale)
    torch.cuda.synchronize()

    nk3 = nk.view(B, Hkv, D)
    nv3 = nv.view(B, Hkv, D)

    def step(pool):
        if fp8 and a.unfused:
            ops.reshape_and_cache_fp8(nk, nv, slots_dev, pool, k_scale, v_scale)
            ops.decode_fp8(out, q, pool, bt_dev, sl_dev, msl, scale, k_scale, v_scale, P, ws,
                           plan=plan_dev)
        elif fp8:   # pa_decode_append_fp8: quantised cache write + decode in one launch
            ops.decode_fp8(out, q, pool, bt_dev, sl_dev, msl, scale, k_scale, v_scale, P, ws,
                           plan=plan_dev, new_key=nk3, new_value=nv3)
        elif a.unfused:
            ops.reshape_and_cache(nk, nv, slots_dev, pool)
            ops.decode(out, q, pool, bt_dev, sl_dev, msl, scale, P, ws, plan=plan_dev)
        else:   # pa_decode_append: cache write + decode in one launch
            ops.decode(out, q, pool, bt_dev, sl_dev, msl, scale, P, ws, plan=plan_dev,
                       new_key=nk3, new_value=nv3)

    def decode_only(pool):
        if fp8 and a.unfused:
            ops.decode_fp8(out, q, pool, bt_dev, sl_dev, msl, scale, k_scale, v_scale, P, ws,
                           plan=plan_dev)
        elif fp8:
            ops.decode_fp8(out, q, pool, bt_dev, sl_dev, msl, scale, k_scale, v_scale, P, ws,
                           plan=plan_dev, new_key=nk3, new_value=nv3)
        elif a.unfused:
            ops.decode(out, q, pool, bt_dev, sl_dev, msl, scale, P, ws, plan=plan_dev)
        else:
            ops.decode(out, q, pool, bt_dev, sl_dev, msl, scale, P, ws, plan=plan_dev,
                       new_key=nk3, new_value=nv3)

    def capture(fn, n):
        """One HIP graph of n calls of fn, call i on pool copy i % R (the pages'
        remedy for launch overhead: pre-recorded work replayed as a whole)."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(min(n, R)):
                fn(pools[i % R])
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(pools[i % R])
        return g

    g_warm = capture(step, max(1, a.warmup))
    g_step = capture(step, a.steps)
    g_dec = capture(decode_only, a.steps)

    # warm-up, then the timed region: exactly `steps` decode steps
    g_warm.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    g_step.replay()
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / a.steps

    # the dominant kernel alone: `steps` decode launches back to back, same rotation
    g_dec.replay()
    torch.cuda.synchronize()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record()
    g_dec.replay()
    d1.record()
    torch.cuda.synchronize()
    dec_us = d0.elapsed_time(d1) * 1e3 / a.steps

    # a plain device copy of 1 GiB for a measured bandwidth beside the
    # nominal peak (read + write bytes per copy; pools already rotated out)
    cbuf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(cbuf)
    cdst.copy_(cbuf)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        cdst.copy_(cbuf)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del cbuf, cdst

    # the same steps launched eagerly from the host (argument checks, ctypes
    # call and dispatch per step), for the launch overhead the graph removes
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for i in range(a.steps):
        step(pools[i % R])
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - h0) * 1e6 / a.steps

    ctx = int(seq_lens.sum())
    kvb = 1 if fp8 else None
    dbytes = decode_bytes(wl, seq_lens, kvb)
    step_bytes = dbytes + cache_write_bytes(wl, kvb)
    kbytes = dbytes if a.unfused else step_bytes   # the timed kernel's own bytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = kbytes / (dec_us * 1e-6) / 1e9
    khash = source_hash(DECODE_SOURCES)
    traffic = None
    if not fp8 and a.workload == 1 and P == 0:
        traffic = load_traffic(khash, a.unfused)
    elif (not fp8 and not a.unfused and a.workload in WORKLOAD_TRAFFIC
          and P == default_partition(wl)):
        traffic = load_traffic(khash, False, WORKLOAD_TRAFFIC[a.workload])
    elif fp8 and not a.unfused and a.workload in FP8_TRAFFIC and P == default_partition(wl):
        traffic = load_traffic(khash, False, FP8_TRAFFIC[a.workload])

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) keys/values/queries; no weights)",
        "config": {
            "workload": wl.name, "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_size": D, "block_size": bs, "context_tokens": ctx, "max_seq_len": msl,
            "partition_size": P, "pool_blocks": d.num_blocks, "pool_copies_rotated": R,
            "kv_cache": ("fp8-e4m3, per-tensor scales k %.6g v %.6g" % (k_scale, v_scale)
                         if fp8 else wl.dtype),
            "parallelism": "none (1 GPU)",
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "context_tokens_per_s": round(ctx / (ms_step * 1e-3), 1),
        "host_metadata_us": round(host_us, 1),            # from scratch: allocator, tables
        "host_step_us": round(step_host_us, 2),           # per step, incremental, one native call
        "host_step_us_python": round(step_host_us_py, 2),  # the same composed in Python
        "step_us_eager_launches": round(eager_us, 2),   # no graph: host launch per step
        "measured_copy_gbs": round(copy_gbs, 1),          # 1 GiB device copy, read + write
        "roofline": {
            "kernel": ("pa_decode_fp8 (decode_kernel, FP8 cache)" if fp8 and a.unfused else
                       "pa_decode_append_fp8 (decode_kernel, FP8 cache, quantised cache write "
                       "fused)" if fp8 else
                       "pa_decode (decode_kernel)" if a.unfused else
                       "pa_decode_append (decode_kernel, cache write fused)"),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kbytes,
            "avg_launch_us": round(dec_us, 3),
            "kernel_source_hash": khash,
        },
    }
    if not a.no_cpu_baseline:
        dt, reps, seqs = cpu_baseline(d, a.cpu_seconds, (k_scale, v_scale) if fp8 else None)
        sub = d.seq_lens[seqs]
        sample_bytes = decode_bytes(wl, sub, kvb) + cache_write_bytes(wl, kvb, len(seqs))
        sctx = int(sub.sum())
        what = (f"the whole {wl.name} step" if len(seqs) == B else
                f"{len(seqs)} of the {B} sequences of the {wl.name} step (seeded choice: "
                f"sequences {seqs}, lengths {[int(x) for x in sub]})")
        res["cpu_baseline"] = {
            "value": round(sample_bytes / dt / 1e9, 4),
            "unit": "GB/s",
            "cores": 1,
            "host_cores": host_cores(),
            "blas_threads": 1,
            "context_tokens_per_s": round(sctx / dt, 1),
            "kind": "oracle",
            "sample": f"{what}: write the new tokens, decode ({sctx} context tokens), "
                      f"repeated {reps}x; fp64 numpy on one core (BLAS 1 thread); "
                      f"{dt * 1e3:.1f} ms per pass",
        }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
