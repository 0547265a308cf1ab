#!/usr/bin/env python3
"""Benchmark: one decode step of PagedAttention at the Llama-3.1-70B layer
shape with an FP8 E4M3 KV cache, on one MI355X.

Workload (the shape of "Optimización de KV Cache con PagedAttention y
Cuantización FP8 ...", §2, at one layer): 64 sequences, 8192 cached tokens
each plus one new token, 64 query / 8 KV heads, head dim 128, 16-token blocks
scattered over a shuffled pool of 36864 blocks, per-tensor scales amax/448.

A step is the whole hot path on one batch: the host assigns the new tokens'
slots (block pool, done once in set-up since it changes the state), then on
the device pkv_reshape_and_cache stores the 64 new K/V rows into their FP8
slots, then the partition kernel attends over L = 8193 tokens per sequence
(split-KV partitions, merged by a second kernel when a sequence spans
several).

Prints one JSON line.  `value` = KV bytes the step must read (every cached
token once, K and V, all KV heads: 1,073,872,896 B) / step time, in GB/s.
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
KERNEL_SRC = os.path.join(ROOT, "paged_kv_cache_270_amd", "csrc", "pkv_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_partition_llama70b_fp8.json")


def kernel_source_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic():
    """HBM bytes per launch of the partition kernel from the committed
    rocprofv3 counter runs, if they were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--cpu-sample-seqs", type=int, default=8,
                    help="sequences of the workload the CPU oracle baseline decodes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB, 5 times (the "
                         "reference kernel for scaling HBM byte counters), then exit")
    args = ap.parse_args()
    if args.copy_probe_mib:
        return copy_probe(args.copy_probe_mib)
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by sequence or KV head with no exchange; see DESIGN.md)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import paged_kv_cache_270_amd as pkv
    from paged_kv_cache_270_amd import workloads

    torch.cuda.set_device(0)
    dev = "cuda"
    B, cached, Hq, Hkv, D, NB = 64, 8192, 64, 8, 128, 36864
    L = cached + 1
    layout = pkv.CacheLayout(NB, Hkv, pkv.PKV_FP8_E4M3FN)

    # ---- a1 on the host: block pool, on-demand allocation, shuffled placement
    pool = pkv.BlockPool(NB, shuffle_seed=3)
    seqs = [pool.create() for _ in range(B)]
    bulk_slots = np.concatenate([np.asarray(pool.append(s, cached)[0]) for s in seqs])
    t0 = time.perf_counter()
    step_slots = np.array([pool.append(s, 1)[0][0] for s in seqs], dtype=np.int64)
    host_slot_us = (time.perf_counter() - t0) * 1e6
    tables = np.stack([np.asarray(pool.block_table(s), dtype=np.int32) for s in seqs])
    assert tables.shape == (B, L // 16 + 1)

    # ---- inputs resident in HBM
    key_src = workloads.randn_f16((B * cached, Hkv, D), 301, dev)
    val_src = workloads.randn_f16((B * cached, Hkv, D), 302, dev)
    new_k = workloads.randn_f16((B, Hkv, D), 303, dev)
    new_v = workloads.randn_f16((B, Hkv, D), 304, dev)
    q = workloads.randn_f16((B, Hq, D), 305, dev)
    k_scale = float(np.float32(max(key_src.abs().max().item(), new_k.abs().max().item())) /
                    np.float32(448))
    v_scale = float(np.float32(max(val_src.abs().max().item(), new_v.abs().max().item())) /
                    np.float32(448))
    k_pool = torch.zeros(pkv.pkv_pool_bytes(layout), dtype=torch.uint8, device=dev)
    v_pool = torch.zeros_like(k_pool)
    d_bulk_slots = torch.from_numpy(bulk_slots.astype(np.int64)).to(dev)
    d_step_slots = torch.from_numpy(step_slots).to(dev)
    d_tables = torch.from_numpy(tables).to(dev)
    d_lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    sm_scale = float(np.float32(1 / np.sqrt(D)))
    P = pkv.pkv_decode_partition_size(B, Hkv, L, layout.dtype, args.partition_size)
    ws = torch.empty(max(1, pkv.pkv_decode_workspace_bytes(B, Hq, Hkv, L, layout.dtype, P)),
                     dtype=torch.uint8, device=dev)

    # ---- bulk fill (prefill-sized write of 524288 tokens), timed on its own
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    pkv.pkv_reshape_and_cache(key_src, val_src, k_pool, v_pool, d_bulk_slots, layout, k_scale,
                              v_scale)
    e1.record()
    torch.cuda.synchronize()
    bulk_ms = e0.elapsed_time(e1)
    bulk_bytes = B * cached * Hkv * D * 2 * (2 + 1) + B * cached * 8   # fp16 in, FP8 out, slots
    del key_src, val_src

    def step(ev=None):
        pkv.pkv_reshape_and_cache(new_k, new_v, k_pool, v_pool, d_step_slots, layout, k_scale,
                                  v_scale)
        if ev is not None:
            ev[0].record()
        pkv.pkv_decode_partitions(out, q, k_pool, v_pool, d_tables, d_lens, L, layout,
                                  sm_scale, k_scale, v_scale, P, ws)
        if ev is not None:
            ev[1].record()
        pkv.pkv_decode_reduce(out, d_lens, L, tables.shape[1], layout, v_scale, P, ws)

    def timed(fn):
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(args.steps):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    for _ in range(args.warmup):
        step()
    # the timed region: K whole steps back to back, nothing else on the stream
    step_ms = timed(step)
    # a second timed region of K steps with events around the partition kernel
    # (same stream) for its own duration; events add a few microseconds per
    # step, so the step time above is taken without them
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(kev[i])
    torch.cuda.synchronize()
    kern_ms = sorted(a.elapsed_time(b) for a, b in kev)
    part_ms = sum(kern_ms) / len(kern_ms)

    kv_bytes = B * L * Hkv * D * 2 * 1
    value = kv_bytes / (step_ms * 1e-3) / 1e9
    achieved = kv_bytes / (part_ms * 1e-3) / 1e9
    traffic = measured_traffic()

    # ---- CPU baseline: the oracle on a bounded sample of the same workload.
    # Its inputs are built on the host by the oracle itself (its own write of
    # freshly drawn rows into the same slots), never copied from the device.
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        S = max(1, min(B, args.cpu_sample_seqs))
        threads = min(os.cpu_count() or 1, 16)
        kh = np.zeros(pkv.pkv_pool_bytes(layout), dtype=np.uint8)
        vh = np.zeros_like(kh)
        n_tok = S * cached
        rng = np.random.default_rng(306)
        src_k = rng.standard_normal((n_tok + S, Hkv, D), dtype=np.float32).astype(np.float16)
        src_v = rng.standard_normal((n_tok + S, Hkv, D), dtype=np.float32).astype(np.float16)
        host_slots = np.concatenate([bulk_slots[:n_tok], step_slots[:S]]).astype(np.int64)
        oracle.reshape_and_cache(src_k, src_v, kh, vh, host_slots, Hkv, True, k_scale, v_scale)
        qh = rng.standard_normal((S, Hq, D), dtype=np.float32).astype(np.float16)
        t0 = time.perf_counter()
        oracle.paged_attention_decode(qh, kh, vh, tables[:S], np.full(S, L, np.int32), Hkv,
                                      True, sm_scale, k_scale, v_scale, threads)
        cpu_s = time.perf_counter() - t0
        cpu = {"value": round(S * L * Hkv * D * 2 / cpu_s / 1e9, 4), "unit": "GB/s",
               "cores": threads, "kind": "oracle",
               "sample": f"{S} of {B} sequences (all 64 query heads, L={L}): "
                         f"{cpu_s:.2f} s fp64 decode on the host"}

    res = {
        "metric": "KV GB/s read (% of HBM peak) + decode seqs·tok/s, 70B-layer shape, FP8 KV",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "llama-3.1-70b layer decode, FP8 E4M3 KV cache",
                   "global_batch": B, "seq_len": L, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "block_size": 16, "pool_blocks": NB, "partition_size": P,
                   "kv_dtype": "fp8_e4m3fn", "arith": "f16 MFMA inputs, f32 accumulate",
                   "parallelism": "single GPU"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_tok_per_s": round(B * L / (step_ms * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
        "decode_partition_us": round(part_ms * 1e3, 2),
        "host_slot_assignment_us": round(host_slot_us, 1),
        "bulk_fill_gbs": round(bulk_bytes / (bulk_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
