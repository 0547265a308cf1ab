#!/usr/bin/env python3
"""Benchmark: one decode step of PagedAttention over a paged FP8 KV cache on one
MI355X.

Default workload (the metric's): the Llama-3.1-70B layer shape of "Optimización
de KV Cache con PagedAttention y Cuantización FP8 ...", §2 -- 64 sequences,
8192 cached tokens each plus one new token, 64 query / 8 KV heads, head dim
128, 16-token blocks scattered over a shuffled pool of 36864 blocks, FP8 E4M3
cache with per-tensor scales amax/448.  `--workload` selects the other
reference shapes (tiny, fp16 batch, 128K contexts, ragged shared prefixes);
`--kv-scales block` switches an FP8 workload to per-(block, KV head) scales
measured as the cache is written (same page, §8, dynamic scaling).

Every workload is built through the library's host block pool: sequences are
created and grown block by block (forked from a group leader where they share
a prefix), cached tokens are written by pkv_reshape_and_cache, and the pool
hands out each sequence's slot for the new token (timed: host_slot_assignment).

A step is the whole hot path on one batch: each sequence's new K/V row is
stored into its slot and the partition kernel attends over L tokens per
sequence -- one launch, pkv_decode_partitions_append, whose kernel also
writes the new rows -- and, when some sequence spans several partitions, the
merge kernel combines them.  With `--kv-scales block` the write is
pkv_reshape_and_cache_dynamic, launched first.  Prints one JSON line;
`value` = KV bytes the step must read from HBM (each stored token once, K and
V, all KV heads) / step time, in GB/s.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BULK_REPS = 7   # timed bulk fills; the median is reported
METRIC = "KV GB/s read (% of HBM peak) + decode seqs·tok/s, 70B-layer shape, FP8 KV"
CSRC = os.path.join(ROOT, "paged_kv_cache_270_amd", "csrc")
# the sources each measured kernel is built from
DECODE_SRCS = ("pkv_kernels.hip", "pkv_tile.h", "pkv_codec.h")
PREFILL_SRCS = ("pkv_prefill.hip", "pkv_tile.h")
TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def kernel_source_sha(sources=DECODE_SRCS) -> str:
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(key: str, sources=DECODE_SRCS):
    """HBM bytes per launch of the measured kernel from committed rocprofv3
    counter runs (profiles/traffic_<key>.json), if taken on the current
    kernel sources."""
    try:
        with open(os.path.join(TRAFFIC_DIR, f"traffic_{key}.json")) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_sha(sources):
        return None
    return t.get("hbm_bytes_per_launch")


CPU_MIN_S = 10.0  # the CPU baseline repeats its sample until this much time has passed


def timed_reps(fn, min_s: float = CPU_MIN_S):
    """Run fn until at least min_s seconds have passed (at least once);
    returns (runs, seconds)."""
    runs, t0 = 0, time.perf_counter()
    while True:
        fn()
        runs += 1
        s = time.perf_counter() - t0
        if s >= min_s:
            return runs, s


def library_gemm_tfs(n: int = 8192, reps: int = 20) -> float:
    """An fp16 n x n x n product through torch.matmul (the ROCm BLAS library):
    the matrix-core rate a vendor-tuned dense kernel reaches on this part,
    next to which the prefill kernel's rate is read."""
    import torch
    a = torch.randn((n, n), dtype=torch.float16, device="cuda")
    b = torch.randn((n, n), dtype=torch.float16, device="cuda")
    for _ in range(3):
        c = torch.matmul(a, b)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        c = torch.matmul(a, b)
    t1.record()
    torch.cuda.synchronize()
    del a, b, c
    return 2.0 * n ** 3 / (t0.elapsed_time(t1) / reps * 1e-3) / 1e12


def copy_probe(mib: int) -> int:
    """A plain copy of known size: reads and writes mib MiB per launch."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_launch": n, "launches": 5}), flush=True)
    return 0


def read_probe(mib: int) -> int:
    """Only the streaming-read ceiling: mib MiB read 20 times after 3 warm-up
    reads, one JSON line with the rate."""
    import torch
    import paged_kv_cache_270_amd as pkv
    torch.cuda.set_device(0)
    gbs = stream_read_gbs(pkv, mib << 20)
    print(json.dumps({"stream_read_bytes_per_launch": mib << 20, "stream_read_gbs": gbs}),
          flush=True)
    return 0


SETTLE_MS = 60.0


def settle(fn, min_ms: float = SETTLE_MS) -> int:
    """Untimed calls of `fn`, in batches of 8, until at least `min_ms` of GPU
    time has passed; returns how many ran.  Run before the W warmup steps:
    after the setup's idle gaps the part takes some milliseconds to come back
    to full speed, longer than a few warmup steps last (the 70B FP8 step
    measured 168-171 us after 10 warmup steps, 163.5-163.8 us after 200)."""
    import torch
    n, spent = 0, 0.0
    while spent < min_ms:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(8):
            fn()
        b.record()
        torch.cuda.synchronize()
        spent += a.elapsed_time(b)
        n += 8
    return n


def timed_launches(fn, reps: int, warmup: int = 3) -> float:
    """Milliseconds per call of `fn` over `reps` back-to-back calls between two
    events on the current stream (nothing else in between)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def stream_read_gbs(pkv, nbytes: int = 2 << 30) -> float:
    """Streaming-read ceiling: a contiguous buffer (far larger than the 256 MB
    last-level cache) read once per launch with 16-byte non-temporal loads,
    the best of four grid sizes."""
    import torch
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    # the best of a few launch shapes (workgroups of 256 lanes, each its own slab)
    ms = min(timed_launches(lambda: pkv.pkv_hbm_read_probe(buf, sink, wg), 20)
             for wg in (1024, 2048, 4096, 8192))
    del buf
    return round(nbytes / (ms * 1e-3) / 1e9, 1)


def write_mix_gbs(pkv, reads_per_write: int, dst_bytes: int = 1 << 30) -> float:
    """Ceiling for a write that reads `reads_per_write` bytes per byte it
    writes (the cache write: 2 for FP8, 1 for fp16): contiguous planes
    streamed into a destination, non-temporal both ways, the best of four grid
    sizes; GB/s counts the bytes read and written."""
    import torch
    src = torch.empty(reads_per_write * dst_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(dst_bytes, dtype=torch.uint8, device="cuda")
    ms = min(timed_launches(lambda: pkv.pkv_hbm_mix_probe(src, dst, reads_per_write, wg), 10)
             for wg in (1024, 2048, 4096, 8192))
    del src, dst
    return round((reads_per_write + 1) * dst_bytes / (ms * 1e-3) / 1e9, 1)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def sha256_of(a) -> str:
    import numpy as np
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def build_sequences(pkv, wl):
    """Grow the workload's sequences in the library's block pool.

    Returns (pool, seq ids, cached-token slots per sequence (a shared prefix
    listed under every member), slots written once (the bulk fill), new-token
    slots, host microseconds spent assigning the new tokens' slots)."""
    import numpy as np
    pool = pkv.BlockPool(wl.num_blocks, shuffle_seed=wl.seed)
    lens = [int(x) for x in wl.context_lens]
    seqs, per_seq, written = [], [], []
    if wl.groups:
        for members in wl.groups:
            leader = pool.create()
            prefix = pool.append(leader, wl.prefix_blocks * 16)[0]
            written.extend(prefix)
            ids = [leader] + [pool.fork(leader) for _ in members[1:]]
            for sid, b in zip(ids, members):
                tail = pool.append(sid, lens[b] - len(prefix) - 1)[0]
                written.extend(tail)
                seqs.append(sid)
                per_seq.append(list(prefix) + tail)
    else:
        for L in lens:
            sid = pool.create()
            got = pool.append(sid, max(L - 1, 0))[0]
            written.extend(got)
            seqs.append(sid)
            per_seq.append(got)
    import gc
    gc.disable()                      # time the appends, not a collection of set-up lists
    pool.append_each([])                        # first call's set-up, nothing appended
    t0 = time.perf_counter()
    step_slots, _ = pool.append_each(seqs)      # one call for the whole batch
    host_us = (time.perf_counter() - t0) * 1e6
    gc.enable()
    return (pool, seqs, per_seq, np.asarray(written, dtype=np.int64),
            np.asarray(step_slots, dtype=np.int64), host_us)


MFMA_F16_PEAK_TFS = 2500.0    # MI355X dense fp16 matrix peak


def run_prefill(args) -> int:
    """One chunked-prefill step: write the chunk's new K/V rows, then causal
    attention of the chunk's queries over the whole paged cache.  `value` is
    algorithmic TFLOP/s (QK^T and PV over every visible token, 4 * D flop per
    token, query row and head) for the attention plus its write."""
    import numpy as np
    import torch

    import paged_kv_cache_270_amd as pkv
    from paged_kv_cache_270_amd import workloads

    torch.cuda.set_device(0)
    dev = "cuda"
    wl = workloads.PREFILL_CONFIGS[args.workload]()
    B, Hq, Hkv, D = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, workloads.D
    layout = pkv.CacheLayout(wl.num_blocks, Hkv, pkv.PKV_FP8_E4M3FN if wl.fp8 else pkv.PKV_F16)
    # the block pool hands out every block: the earlier tokens, then the chunk
    pool = pkv.BlockPool(wl.num_blocks, shuffle_seed=wl.seed)
    seqs, early, chunk = [], [], []
    for L, n in zip(wl.context_lens.tolist(), wl.chunk_lens.tolist()):
        sid = pool.create()
        early.extend(pool.append(sid, L - n)[0])
        chunk.extend(pool.append(sid, n)[0])
        seqs.append(sid)
    rows = [pool.block_table(s) for s in seqs]
    tables = np.zeros((B, max(len(r) for r in rows)), dtype=np.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = r
    Te, Tc = len(early), len(chunk)
    dyn = args.kv_scales == "block"
    if dyn and not wl.fp8:
        print("bench.py: per-block scales apply to FP8 caches only", file=sys.stderr)
        return 2
    ks, vs = (0.011, 0.013) if wl.fp8 else (1.0, 1.0)   # N(0,1) rows stay far below 448 * scale
    k_pool = torch.zeros(pkv.pkv_pool_bytes(layout), dtype=torch.uint8, device=dev)
    v_pool = torch.zeros_like(k_pool)
    if dyn:   # per-(block, KV head) scales, measured as the cache is written
        k_bs = torch.zeros((wl.num_blocks, Hkv), dtype=torch.float32, device=dev)
        v_bs = torch.zeros_like(k_bs)
        ws = torch.empty(pkv.pkv_reshape_dynamic_workspace_bytes(layout), dtype=torch.uint8,
                         device=dev)

    def write(k, v, slots):
        if dyn:
            pkv.pkv_reshape_and_cache_dynamic(k, v, k_pool, v_pool, k_bs, v_bs, slots, layout, ws)
        else:
            pkv.pkv_reshape_and_cache(k, v, k_pool, v_pool, slots, layout, ks, vs)

    if Te:
        write(workloads.randn_f16((Te, Hkv, D), 401, dev),
              workloads.randn_f16((Te, Hkv, D), 402, dev),
              torch.from_numpy(np.asarray(early, np.int64)).to(dev))
    new_k = workloads.randn_f16((Tc, Hkv, D), 403, dev)
    new_v = workloads.randn_f16((Tc, Hkv, D), 404, dev)
    q = workloads.randn_f16((Tc, Hq, D), 405, dev)
    d_chunk = torch.from_numpy(np.asarray(chunk, np.int64)).to(dev)
    d_tables = torch.from_numpy(tables).to(dev)
    d_lens = torch.from_numpy(wl.context_lens).to(dev)
    d_qs = torch.from_numpy(wl.query_start).to(dev)
    out = torch.empty((Tc, Hq, D), dtype=torch.float32, device=dev)
    sm = float(np.float32(1 / np.sqrt(D)))
    maxq, maxl = int(wl.chunk_lens.max()), int(wl.context_lens.max())

    def attention():
        if dyn:
            pkv.pkv_paged_prefill_attention_dynamic(out, q, k_pool, v_pool, k_bs, v_bs, d_tables,
                                                    d_lens, d_qs, maxq, maxl, layout, sm)
        else:
            pkv.pkv_paged_prefill_attention(out, q, k_pool, v_pool, d_tables, d_lens, d_qs, maxq,
                                            maxl, layout, sm, ks, vs)

    def step():
        write(new_k, new_v, d_chunk)
        attention()

    settle_steps = settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / args.steps
    # the attention kernel alone: K back-to-back launches, no event between
    attn_ms = min(timed_launches(attention, args.steps, warmup=1), step_ms)
    flops = wl.flops()
    value = flops / (step_ms * 1e-3) / 1e12
    achieved = flops / (attn_ms * 1e-3) / 1e12
    gemm_tfs = library_gemm_tfs()

    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on a bounded sample: a few chunk rows, each as a one-token
        # chunk over its prefix, on inputs the oracle writes itself
        import oracle
        rng = np.random.default_rng(406)
        S = max(1, args.cpu_sample_seqs // 16)
        b = B - 1
        L, n = int(wl.context_lens[b]), int(wl.chunk_lens[b])
        kh = np.zeros(pkv.pkv_pool_bytes(layout), dtype=np.uint8)
        vh = np.zeros_like(kh)
        sl = np.asarray(pool.block_table(seqs[b]), np.int64)
        pos = np.arange(L)
        slots = sl[pos // 16] * 16 + pos % 16
        src = rng.standard_normal((L, Hkv, D), dtype=np.float32).astype(np.float16)
        if dyn:
            ksh = np.zeros((wl.num_blocks, Hkv), np.float32)
            vsh = np.zeros_like(ksh)
            oracle.reshape_and_cache_dynamic(src, src, kh, vh, ksh, vsh, slots, Hkv)
        else:
            oracle.reshape_and_cache(src, src, kh, vh, slots, Hkv, wl.fp8, ks, vs)
        qh = rng.standard_normal((S, Hq, D), dtype=np.float32).astype(np.float16)
        threads = min(os.cpu_count() or 1, 16)
        ps = [L - 1 - 97 * i for i in range(S)]

        def rows():
            for i, p in enumerate(ps):
                if dyn:
                    oracle.paged_prefill_attention_dynamic(qh[i:i + 1], kh, vh, ksh, vsh,
                                                           tables[b:b + 1], [p + 1], [0, 1],
                                                           Hkv, sm, threads)
                else:
                    oracle.paged_prefill_attention(qh[i:i + 1], kh, vh, tables[b:b + 1],
                                                   [p + 1], [0, 1], Hkv, wl.fp8, sm, ks, vs,
                                                   threads)
        runs, cpu_s = timed_reps(rows)
        sample_flops = sum(p + 1 for p in ps) * Hq * 4 * D
        cpu = {"value": round(runs * sample_flops / cpu_s / 1e12, 6), "unit": "TFLOP/s",
               "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"{S} chunk rows near position {L - 1} of the deepest sequence (all "
                         f"{Hq} query heads), computed {runs} times: {cpu_s:.2f} s fp64 on "
                         f"the host"}

    res = {
        "metric": "chunked-prefill attention TFLOP/s (algorithmic), 70B-layer shape",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "global_batch": B, "chunk_tokens": int(Tc),
                   "seq_len": maxl, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                   "block_size": 16, "pool_blocks": wl.num_blocks,
                   "kv_dtype": "fp8_e4m3fn" if wl.fp8 else "f16",
                   "kv_scales": ("per (block, kv head)" if dyn else "per tensor") if wl.fp8
                   else None,
                   "arith": "f16 MFMA inputs, f32 accumulate, f16 probabilities",
                   "parallelism": "single GPU"},
        "flops_per_step": flops,
        "prefill_attention_ms": round(attn_ms, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFS, 4),
                     "traffic": measured_traffic("prefill_" + args.workload +
                                                 ("_block_scales" if dyn else ""),
                                                 PREFILL_SRCS)},
        "mfma_ceilings": {"library_f16_gemm_tfs": round(gemm_tfs, 1),
                          "library_gemm": "torch.matmul, fp16 8192 x 8192 x 8192",
                          "kernel_frac_of_library_gemm": round(achieved / gemm_tfs, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


def run_swap(args) -> int:
    """Page-granular eviction: a quarter of the 70B-layer FP8 batch's pages
    (16 sequences x 513 blocks, all KV heads, K and V) go to pinned host
    memory and come back.  `value` = bytes moved per direction / copy time
    (GB/s), the mean of the two directions; the pool bookkeeping is timed on
    the host separately.  A plain DMA copy of the same bytes between pinned
    host and device memory is timed as the link's ceiling."""
    import numpy as np
    import torch

    import paged_kv_cache_270_amd as pkv
    from paged_kv_cache_270_amd import workloads

    torch.cuda.set_device(0)
    dev = "cuda"
    wl = workloads.llama70b_fp8()
    B, Hkv, D, NB = wl.num_seqs, wl.num_kv_heads, workloads.D, wl.num_blocks
    layout = pkv.CacheLayout(NB, Hkv, pkv.PKV_FP8_E4M3FN)
    pool, seqs, per_seq, bulk_slots, step_slots, _ = build_sequences(pkv, wl)
    k_pool = torch.zeros(pkv.pkv_pool_bytes(layout), dtype=torch.uint8, device=dev)
    v_pool = torch.zeros_like(k_pool)
    T = int(bulk_slots.size)
    pkv.pkv_reshape_and_cache(workloads.randn_f16((T, Hkv, D), 301, dev),
                              workloads.randn_f16((T, Hkv, D), 302, dev), k_pool, v_pool,
                              torch.from_numpy(bulk_slots).to(dev), layout, 0.011, 0.013)
    victims = seqs[:16]
    per_block = Hkv * 16 * D            # bytes of one block per pool (FP8)
    H = sum(len(pool.block_table(s)) for s in victims)
    pool.set_swap_space(H)
    host_k = torch.empty(H * per_block, dtype=torch.uint8, pin_memory=True)
    host_v = torch.empty(H * per_block, dtype=torch.uint8, pin_memory=True)
    for s in victims:                    # one untimed round trip warms the pool's lists
        pool.swap_out(s, 0, len(pool.block_table(s)))
    for s in victims:
        pool.swap_in(s)
    import gc
    gc.disable()
    t0 = time.perf_counter()
    out_pairs = [p for s in victims for p in pool.swap_out(s, 0, len(pool.block_table(s)))]
    host_out_us = (time.perf_counter() - t0) * 1e6
    t0 = time.perf_counter()
    in_pairs = [p for s in victims for p in pool.swap_in(s)]
    host_in_us = (time.perf_counter() - t0) * 1e6
    gc.enable()
    assert len(in_pairs) == len(out_pairs) == H
    d_out = torch.tensor(out_pairs, dtype=torch.int32, device=dev)
    # the copies move the same blocks back into the blocks they left (the
    # pool may choose others; the bytes moved are the same)
    d_in = torch.tensor([(h, d) for d, h in out_pairs], dtype=torch.int32, device=dev)
    moved = 2 * H * per_block            # K and V

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    d2h_ms = timed(lambda: pkv.pkv_swap_blocks(k_pool, v_pool, host_k, host_v, H, layout, d_out,
                                               to_host=True))
    h2d_ms = timed(lambda: pkv.pkv_swap_blocks(k_pool, v_pool, host_k, host_v, H, layout, d_in,
                                               to_host=False))
    dma_src = torch.empty(moved, dtype=torch.uint8, device=dev)
    dma_host = torch.empty(moved, dtype=torch.uint8, pin_memory=True)
    dma_d2h = timed(lambda: dma_host.copy_(dma_src, non_blocking=True))
    dma_h2d = timed(lambda: dma_src.copy_(dma_host, non_blocking=True))
    d2h, h2d = moved / (d2h_ms * 1e-3) / 1e9, moved / (h2d_ms * 1e-3) / 1e9
    ceiling = max(moved / (dma_d2h * 1e-3) / 1e9, moved / (dma_h2d * 1e-3) / 1e9)
    value = (d2h + h2d) / 2
    res = {
        "metric": "KV page swap GB/s per direction (device <-> pinned host), 70B-layer FP8 pages",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(d2h_ms + h2d_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": "swap-fp8-16x513-blocks", "blocks": H, "bytes_per_direction": moved,
                   "kv_dtype": "fp8_e4m3fn", "parallelism": "single GPU"},
        "device_to_host_gbs": round(d2h, 2), "host_to_device_gbs": round(h2d, 2),
        "dma_copy_ceiling_gbs": round(ceiling, 2),
        "host_bookkeeping_us": {"swap_out": round(host_out_us, 1), "swap_in": round(host_in_us, 1)},
        "roofline": {"bound": "host-link", "achieved": round(value, 2), "peak": round(ceiling, 2),
                     "unit": "GB/s", "frac": round(value / ceiling, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama70b_fp8",
                    help="llama70b_fp8 (default) | llama70b_fp8_tp4 | llama70b_fp16 | "
                         "long_context | shared_prefix | tiny | prefill_128k | prefill_mixed | "
                         "prefill_128k_fp16 | swap")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="longest split-KV partition in tokens (default: the workload's "
                         "own, else the library's choice)")
    ap.add_argument("--kv-scales", choices=("tensor", "block"), default="tensor",
                    help="FP8 scales: one per tensor (amax/448, default) or one per "
                         "(block, KV head) measured as the cache is written")
    ap.add_argument("--cpu-sample-seqs", type=int, default=64,
                    help="sequences of the workload the CPU oracle baseline decodes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tail-map", choices=("on", "off"), default="on",
                    help="cascade: pass the host pool's list of tail units (on) or let "
                         "each workgroup find its unit by a scan over the lengths (off)")
    ap.add_argument("--cascade", choices=("auto", "on", "off"), default="auto",
                    help="decode each group's shared prefix once for the group "
                         "(pkv_paged_attention_decode_cascade[_dynamic]); auto = when the "
                         "host pool finds prefix groups in the batch")
    ap.add_argument("--graph", action="store_true",
                    help="replay the decode step as one captured HIP graph instead of "
                         "launching its kernels one by one")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB, 5 times (the "
                         "reference kernel for scaling HBM byte counters), then exit")
    ap.add_argument("--read-probe-mib", type=int, default=0,
                    help="only measure the streaming-read ceiling over this many MiB, "
                         "then exit")
    args = ap.parse_args()
    if args.copy_probe_mib:
        return copy_probe(args.copy_probe_mib)
    if args.read_probe_mib:
        return read_probe(args.read_probe_mib)
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by sequence or KV head with no exchange; see DESIGN.md)",
              file=sys.stderr)
        return 2

    from paged_kv_cache_270_amd import workloads as _wls
    if args.workload in _wls.PREFILL_CONFIGS:
        return run_prefill(args)
    if args.workload == "swap":
        return run_swap(args)

    import numpy as np
    import torch

    import paged_kv_cache_270_amd as pkv
    from paged_kv_cache_270_amd import workloads

    torch.cuda.set_device(0)
    dev = "cuda"
    wl = workloads.CONFIGS[args.workload]()
    B, Hq, Hkv, D, NB = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, workloads.D, wl.num_blocks
    Lmax = wl.max_context_len
    e = wl.elem_bytes
    layout = pkv.CacheLayout(NB, Hkv, pkv.PKV_FP8_E4M3FN if wl.fp8 else pkv.PKV_F16)
    dyn = args.kv_scales == "block"
    if dyn and not wl.fp8:
        print("bench.py: per-block scales apply to FP8 caches only", file=sys.stderr)
        return 2

    # ---- a1 on the host: block pool, on-demand allocation, forks, shuffled placement
    pool, seqs, per_seq, bulk_slots, step_slots, host_slot_us = build_sequences(pkv, wl)
    lens = np.array([pool.seq_len(s) for s in seqs], dtype=np.int32)
    assert np.array_equal(lens, wl.context_lens)
    rows = [pool.block_table(s) for s in seqs]
    # cache hint: leading blocks each sequence shares with others (refcount > 1)
    shared = np.array([pool.shared_prefix_blocks(s) for s in seqs], dtype=np.int32)
    tables = np.zeros((B, max(len(r) for r in rows)), dtype=np.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = r

    # ---- inputs resident in HBM
    T = int(bulk_slots.size)
    key_src = workloads.randn_f16((T, Hkv, D), 301, dev)
    val_src = workloads.randn_f16((T, Hkv, D), 302, dev)
    new_k = workloads.randn_f16((B, Hkv, D), 303, dev)
    new_v = workloads.randn_f16((B, Hkv, D), 304, dev)
    q = workloads.randn_f16((B, Hq, D), 305, dev)
    if wl.fp8:
        k_scale = float(np.float32(max(key_src.abs().max().item(), new_k.abs().max().item())) /
                        np.float32(448))
        v_scale = float(np.float32(max(val_src.abs().max().item(), new_v.abs().max().item())) /
                        np.float32(448))
    else:
        k_scale = v_scale = 1.0
    k_pool = torch.zeros(pkv.pkv_pool_bytes(layout), dtype=torch.uint8, device=dev)
    v_pool = torch.zeros_like(k_pool)
    d_bulk_slots = torch.from_numpy(bulk_slots).to(dev)
    d_step_slots = torch.from_numpy(step_slots).to(dev)
    d_tables = torch.from_numpy(tables).to(dev)
    d_lens = torch.from_numpy(lens).to(dev)
    d_shared = torch.from_numpy(shared).to(dev) if shared.any() else None
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    sm_scale = float(np.float32(1 / np.sqrt(D)))
    req = wl.partition_size if args.partition_size is None else args.partition_size
    P = pkv.pkv_decode_partition_size(B, Hkv, Lmax, layout.dtype, req)
    # prefix groups of the batch, found by the host pool from the forks
    prefix, garr, max_pre, order = pool.prefix_groups(seqs, 8, with_order=True)
    cascade = args.cascade == "on" or (args.cascade == "auto" and garr.shape[0] > 0)
    # the library's vector-ALU decode kernel (an environment switch read by
    # the library) covers FP8 per-tensor decode of groups of at most 8 heads
    valu = (os.environ.get("PKV_DECODE_MATH") == "valu" and wl.fp8 and not dyn and not cascade
            and Hq // Hkv <= 8)
    tail_units = 0
    if cascade:
        d_prefix = torch.from_numpy(prefix).to(dev)
        d_groups = torch.from_numpy(garr).to(dev) if garr.shape[0] else None
        d_order = torch.from_numpy(order).to(dev)   # longest tails first
        # the tail work the launch holds, counted by the pool from its lengths,
        # and (by default) the list of those units, so that no workgroup
        # searches the batch for its own
        tail_units = pool.cascade_tail_units(seqs, prefix, max_pre, P)
        d_tail_map = None
        if args.tail_map == "on":
            d_tail_map = torch.from_numpy(
                pool.cascade_tail_map(seqs, prefix, max_pre, P, order)).to(dev)
        ws_bytes = pkv.pkv_decode_cascade_workspace_bytes(B, Hq, Hkv, Lmax, max_pre,
                                                          layout.dtype, P)
    else:
        ws_bytes = pkv.pkv_decode_workspace_bytes(B, Hq, Hkv, Lmax, layout.dtype, P)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)
    if dyn:
        k_bs = torch.zeros((NB, Hkv), dtype=torch.float32, device=dev)
        v_bs = torch.zeros_like(k_bs)
        wws = torch.empty(pkv.pkv_reshape_dynamic_workspace_bytes(layout), dtype=torch.uint8,
                          device=dev)

    def write(k, v, slots):
        if dyn:
            pkv.pkv_reshape_and_cache_dynamic(k, v, k_pool, v_pool, k_bs, v_bs, slots, layout,
                                              wws)
        else:
            pkv.pkv_reshape_and_cache(k, v, k_pool, v_pool, slots, layout, k_scale, v_scale)

    # ---- bulk fill (a prefill-sized write of every cached token), timed on its
    # own: the first fill loads the kernel and fills the pool, the next ones
    # (same bytes again; every block starts at offset 0, so it is fresh again)
    # are timed one by one and the median is reported
    write(key_src, val_src, d_bulk_slots)
    torch.cuda.synchronize()
    bulk_times = []
    for _ in range(BULK_REPS):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        write(key_src, val_src, d_bulk_slots)
        e1.record()
        torch.cuda.synchronize()
        bulk_times.append(e0.elapsed_time(e1))
    bulk_ms = float(np.median(bulk_times))
    print("bulk fill ms per launch: " + " ".join(f"{t:.3f}" for t in bulk_times),
          file=sys.stderr)
    bulk_bytes = T * Hkv * D * 2 * (2 + e) + T * 8   # fp16 rows in, cache rows out, slots
    del key_src, val_src

    def step():
        if dyn:
            # the newest rows first (the dynamic write's own launch), then
            # one decode call: the partition kernel, and the merge when a
            # sequence spans several partitions (none at the default workload)
            write(new_k, new_v, d_step_slots)
            if cascade:
                pkv.pkv_paged_attention_decode_cascade_dynamic(
                    out, q, k_pool, v_pool, k_bs, v_bs, d_tables, d_lens, Lmax, layout, sm_scale,
                    d_prefix, d_groups, max_pre, P, ws, shared_prefix_blocks=d_shared,
                    seq_order=d_order, tail_units=tail_units,
                    tail_map=d_tail_map)
            else:
                pkv.pkv_paged_attention_decode_dynamic(out, q, k_pool, v_pool, k_bs, v_bs,
                                                       d_tables, d_lens, Lmax, layout, sm_scale,
                                                       P, ws, shared_prefix_blocks=d_shared)
            return
        if cascade:
            # one call: the partition kernel (prefix items and tails, writing
            # the newest tokens), then the merge
            pkv.pkv_paged_attention_decode_cascade(
                out, q, new_k, new_v, k_pool, v_pool, d_tables, d_lens, Lmax, layout, sm_scale,
                d_prefix, d_groups, max_pre, k_scale, v_scale, P, ws,
                shared_prefix_blocks=d_shared, seq_order=d_order, tail_units=tail_units,
                tail_map=d_tail_map)
            return
        # the newest token of each sequence (position L - 1, the slot
        # pool.append gave it) is written by the partition kernel itself
        pkv.pkv_decode_partitions_append(out, q, new_k, new_v, k_pool, v_pool, d_tables, d_lens,
                                         Lmax, layout, sm_scale, k_scale, v_scale, P, ws,
                                         shared_prefix_blocks=d_shared)
        pkv.pkv_decode_reduce(out, d_lens, Lmax, tables.shape[1], layout, v_scale, P, ws)

    def timed(fn):
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(args.steps):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    settle_steps = settle(step)
    for _ in range(args.warmup):
        step()
    # optionally the step as one HIP graph (write, partitions, merge),
    # replayed; measured slower than launching the three kernels here
    run = step
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        run = graph.replay
    # the timed region: K whole steps back to back, nothing else on the stream
    step_ms = timed(run)
    # the dominant kernel's own time, with no event between its launches:
    # where the step is one launch of the partition kernel, the step's timed
    # region is exactly that kernel's; otherwise K back-to-back launches of
    # the partition kernel alone (the per-block-scale decode and the cascade
    # have no entry point for their partition kernel alone: there the decode
    # call -- partitions, and the merge when one is needed -- is timed)
    need_merge = ws_bytes > 0
    if not dyn and not cascade and not need_merge:
        part_ms = step_ms
        part_covers = "partition kernel (the step is one launch of it: the step's timed region)"
    else:
        if dyn and cascade:
            def kernel_only():
                pkv.pkv_paged_attention_decode_cascade_dynamic(
                    out, q, k_pool, v_pool, k_bs, v_bs, d_tables, d_lens, Lmax, layout,
                    sm_scale, d_prefix, d_groups, max_pre, P, ws, shared_prefix_blocks=d_shared,
                    seq_order=d_order, tail_units=tail_units,
                    tail_map=d_tail_map)
            part_covers = "partition + merge kernels (the cascade decode call)"
        elif dyn:
            def kernel_only():
                pkv.pkv_paged_attention_decode_dynamic(out, q, k_pool, v_pool, k_bs, v_bs,
                                                       d_tables, d_lens, Lmax, layout, sm_scale,
                                                       P, ws, shared_prefix_blocks=d_shared)
            part_covers = "partition kernel" + (" + merge" if need_merge else "") + \
                " (the decode call, without the separate write launch)"
        elif cascade:
            def kernel_only():
                pkv.pkv_paged_attention_decode_cascade(
                    out, q, new_k, new_v, k_pool, v_pool, d_tables, d_lens, Lmax, layout,
                    sm_scale, d_prefix, d_groups, max_pre, k_scale, v_scale, P, ws,
                    shared_prefix_blocks=d_shared, seq_order=d_order, tail_units=tail_units,
                tail_map=d_tail_map)
            part_covers = "partition + merge kernels (the cascade call)"
        else:
            def kernel_only():
                pkv.pkv_decode_partitions_append(out, q, new_k, new_v, k_pool, v_pool, d_tables,
                                                 d_lens, Lmax, layout, sm_scale, k_scale,
                                                 v_scale, P, ws, shared_prefix_blocks=d_shared)
            part_covers = "partition kernel (K back-to-back launches of it alone)"
        part_ms = timed_launches(kernel_only, args.steps, warmup=2)
        if part_ms > step_ms:   # timing noise: never report the kernel faster than measured
            print(f"bench.py: kernel-only region {part_ms * 1e3:.2f} us > step "
                  f"{step_ms * 1e3:.2f} us; the step time is used for the roofline",
                  file=sys.stderr)
            part_ms = step_ms
            part_covers += "; bounded by the step time"

    tokens = int(lens.astype(np.int64).sum())
    logical = tokens * Hkv * D * 2 * e                  # every token of every sequence
    unique = (T + B) * Hkv * D * 2 * e                  # each stored token once
    # ---- memory ceilings on the same part: a contiguous streaming read, and
    # the decode's own table-driven tile reads without arithmetic
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    gather_ms = timed_launches(lambda: pkv.pkv_tile_gather_probe(k_pool, v_pool, d_tables, d_lens,
                                                                 Lmax, layout, sink), args.steps)
    gather_gbs = logical / (gather_ms * 1e-3) / 1e9
    stream_gbs = stream_read_gbs(pkv)
    mix_rpw = 2 // e                                    # fp16 rows in per cache byte out
    mix_gbs = write_mix_gbs(pkv, mix_rpw)
    # ---- bytes besides the KV tiles: queries, outputs, table entries and
    # lengths read, the newest rows in and out, split-KV partials written and
    # read back by the merge (max and sum, 128 floats)
    pb = P // 16
    nblk_b = -(-lens.astype(np.int64) // 16)
    if cascade:
        S = np.where((prefix > 0) & (prefix <= max_pre) & (16 * prefix.astype(np.int64) < lens),
                     prefix, 0).astype(np.int64)
        parts = -(-S // pb) + -(-(nblk_b - S) // pb)
    else:
        parts = -(-nblk_b // pb)
    partial_rows = int(np.where(parts > 1, parts, 0).sum()) * Hq
    other = {"q": B * Hq * D * 2, "out": B * Hq * D * 4, "table_entries": int(nblk_b.sum()) * 4,
             "context_lens": B * 4, "new_rows_in": B * Hkv * D * 2 * 2,
             "new_rows_out": B * Hkv * D * e * 2,
             "partials_written_and_read": 2 * partial_rows * (2 + D) * 4}
    if dyn:  # plus one K and one V fp32 scale per (block, KV head) tile read
        nblk = -(-lens.astype(np.int64) // 16)
        used = np.unique(np.concatenate([tables[i, :nblk[i]] for i in range(B)]))
        logical += int(nblk.sum()) * Hkv * 8
        unique += int(used.size) * Hkv * 8
    value = unique / (step_ms * 1e-3) / 1e9
    achieved = unique / (part_ms * 1e-3) / 1e9

    # ---- CPU baseline: the oracle on a bounded sample of the same workload.
    # Its inputs are built on the host by the oracle itself (its own write of
    # freshly drawn rows into the sampled sequences' slots), never copied from
    # the device.
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        S = max(1, min(B, args.cpu_sample_seqs))
        threads = min(os.cpu_count() or 1, 16)
        kh = np.zeros(pkv.pkv_pool_bytes(layout), dtype=np.uint8)
        vh = np.zeros_like(kh)
        slots = np.unique(np.concatenate([np.asarray(per_seq[b], dtype=np.int64)
                                          for b in range(S)] + [step_slots[:S]]))
        rng = np.random.default_rng(306)
        src_k = rng.standard_normal((slots.size, Hkv, D), dtype=np.float32).astype(np.float16)
        src_v = rng.standard_normal((slots.size, Hkv, D), dtype=np.float32).astype(np.float16)
        if not dyn:
            oracle.reshape_and_cache(src_k, src_v, kh, vh, slots, Hkv, wl.fp8, k_scale, v_scale)
        qh = rng.standard_normal((S, Hq, D), dtype=np.float32).astype(np.float16)
        if dyn:
            ksh = np.zeros((NB, Hkv), dtype=np.float32)
            vsh = np.zeros_like(ksh)
            oracle.reshape_and_cache_dynamic(src_k, src_v, kh, vh, ksh, vsh, slots, Hkv)
            runs, cpu_s = timed_reps(lambda: oracle.paged_attention_decode_dynamic(
                qh, kh, vh, ksh, vsh, tables[:S], lens[:S], Hkv, sm_scale, threads))
        else:
            runs, cpu_s = timed_reps(lambda: oracle.paged_attention_decode(
                qh, kh, vh, tables[:S], lens[:S], Hkv, wl.fp8, sm_scale, k_scale, v_scale,
                threads))
        sample_bytes = int(lens[:S].astype(np.int64).sum()) * Hkv * D * 2 * e
        cpu = {"value": round(runs * sample_bytes / cpu_s / 1e9, 4), "unit": "GB/s",
               "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"{S} of {B} sequences (all {Hq} query heads, "
                         f"{int(lens[:S].sum())} tokens), decoded {runs} times: {cpu_s:.2f} s "
                         f"fp64 on the host"}

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name + ("-block-scales" if dyn else ""),
                   "global_batch": B, "seq_len": Lmax,
                   "total_tokens": tokens, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                   "block_size": 16, "pool_blocks": NB, "partition_size": P,
                   "kv_dtype": "fp8_e4m3fn" if wl.fp8 else "f16",
                   "kv_scales": ("per (block, kv head)" if dyn else "per tensor")
                   if wl.fp8 else None,
                   "arith": "f16 2-element dot products (QK^T) and f32 FMAs (PV) on the "
                            "vector ALUs" if valu else "f16 MFMA inputs, f32 accumulate",
                   "parallelism": "single GPU",
                   "launch": "hip graph" if args.graph else "eager",
                   "new_token_write": "separate launch" if dyn else "in the decode kernel",
                   "decode": ("cascade: each shared prefix once per group "
                              f"({garr.shape[0]} groups, {max_pre} prefix blocks, "
                              f"{tail_units} tail units"
                              f"{', listed by the host' if args.tail_map == 'on' else ''})")
                   if cascade else "per sequence"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_tok_per_s": round(tokens / (step_ms * 1e-3), 1),
        "kv_bytes_per_step": unique,
        "kv_bytes_per_step_logical": logical,
        "kv_gbs_logical": round(logical / (step_ms * 1e-3) / 1e9, 2),
        "decode_partition_us": round(part_ms * 1e3, 2),
        "decode_partition_us_covers": part_covers,
        "hbm_ceilings": {"stream_read_gbs": stream_gbs,
                         "tile_gather_gbs": round(gather_gbs, 1),
                         "tile_gather_bytes": logical - (0 if not dyn else
                                                         int(nblk_b.sum()) * Hkv * 8),
                         "value_frac_of_stream_read": round(value / stream_gbs, 4),
                         "kernel_frac_of_stream_read": round(achieved / stream_gbs, 4),
                         "write_mix_gbs": mix_gbs, "write_mix_reads_per_write": mix_rpw,
                         "bulk_fill_frac_of_write_mix":
                             round(bulk_bytes / (bulk_ms * 1e-3) / 1e9 / mix_gbs, 4)},
        "other_bytes_per_step": other,
        "inputs": {"structure_seed": wl.seed, "value_seeds": [301, 302, 303, 304, 305],
                   "context_lens_sha256": sha256_of(lens),
                   "block_tables_sha256": sha256_of(tables)},
        "shared_prefix_blocks_hint": int(shared.max()) if B else 0,
        "host_slot_assignment_us": round(host_slot_us, 1),
        "bulk_fill_gbs": round(bulk_bytes / (bulk_ms * 1e-3) / 1e9, 1),
        "bulk_fill_gbs_range": [round(bulk_bytes / (t * 1e-3) / 1e9, 1)
                                for t in (max(bulk_times), min(bulk_times))],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     # counters were taken at the workload's own partition size,
                     # on the matrix-core kernels
                     "traffic": measured_traffic("decode_partition_" + args.workload +
                                                 ("_block_scales" if dyn else "") +
                                                 ("_cascade" if cascade else ""))
                     if args.partition_size is None and not valu else None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
