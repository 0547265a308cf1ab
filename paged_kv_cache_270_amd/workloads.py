"""Seeded synthetic workloads for tests and the benchmark.

Structure only — sequence lengths, block placement, seeds, value draws.  No
step of the method is computed here: slots are derived from the tables by the
callers (through the library or the oracle), FP8 codes by the library's write
or the oracle's encoder.  Values are N(0, 1) drawn in fp32 and cast to fp16.

Shapes follow the pages' Llama-3.1-70B example ("Optimización de KV Cache con
PagedAttention y Cuantización FP8 ...", §2: 8 KV heads shared 8:1 by 64 query
heads, head dim 128) at one layer, 16-token blocks ("LLM Primer VI,
Capítulo 8", §8.1), and the 128K contexts of the same page (§1).  Physical
blocks are drawn from a shuffled pool, so every table is scattered.
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BS = 16
D = 128


@dataclass
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    fp8: bool
    num_blocks: int
    context_lens: np.ndarray            # int32 [B]: tokens attended (incl. the new one)
    block_tables: np.ndarray            # int32 [B][max_blocks]
    partition_size: int = 0             # 0 = library choice
    # tokens written by the decode step before attention: (sequence, position)
    new_tokens: List[tuple] = field(default_factory=list)
    groups: Optional[List[List[int]]] = None   # sequences sharing a prefix
    prefix_blocks: int = 0

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def elem_bytes(self) -> int:
        return 1 if self.fp8 else 2

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes one decode step reads: every token of every
        sequence once, K and V, all KV heads (GQA: not once per query head)."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * D * 2 * \
            self.elem_bytes

    def unique_kv_bytes(self) -> int:
        """KV bytes of the distinct physical blocks the step touches."""
        seen = set()
        total = 0
        for b in range(self.num_seqs):
            L = int(self.context_lens[b])
            for j in range(-(-L // BS)):
                blk = int(self.block_tables[b, j])
                if blk in seen:
                    continue
                seen.add(blk)
                total += min(BS, L - j * BS)
        return total * self.num_kv_heads * D * 2 * self.elem_bytes

    def pool_elems(self) -> int:
        return self.num_blocks * self.num_kv_heads * BS * D


def _pad_tables(rows, min_width=1):
    width = max(min_width, max((len(r) for r in rows), default=1))
    bt = np.zeros((len(rows), width), dtype=np.int32)
    for i, r in enumerate(rows):
        bt[i, :len(r)] = r
    return bt


def tiny(seed: int = 1, fp8: bool = False, partition_size: int = 0) -> Workload:
    """4 sequences, lengths uniform in [1, 256], 8 query / 2 KV heads, a pool
    of 128 blocks placed by a random permutation, in sequence order."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 257, size=4).astype(np.int32)
    perm = rng.permutation(128).astype(np.int32)
    rows, pos = [], 0
    for L in lens:
        n = -(-int(L) // BS)
        rows.append(perm[pos:pos + n])
        pos += n
    return Workload("tiny", seed, 8, 2, fp8, 128, lens, _pad_tables(rows),
                    partition_size=partition_size)


def llama70b_fp16(seed: int = 2) -> Workload:
    """Batch 32 x 4096 tokens, 64 q / 8 KV heads, fp16 KV, pool of exactly
    8192 blocks shuffled into the tables."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(8192).astype(np.int32).reshape(32, 256)
    lens = np.full(32, 4096, dtype=np.int32)
    return Workload("llama70b-fp16-b32-l4096", seed, 64, 8, False, 8192, lens, perm)


def llama70b_fp8(seed: int = 3, batch: int = 64, cached: int = 8192) -> Workload:
    """Batch 64, 8192 cached tokens each plus one new token per sequence
    written into a freshly taken random free block, so L = 8193; FP8 KV.
    Pool of 36864 blocks, free list shuffled."""
    rng = np.random.default_rng(seed)
    nb = 36864
    free = list(rng.permutation(nb).astype(np.int32))
    per = cached // BS
    rows = [free[b * per:(b + 1) * per] for b in range(batch)]
    taken = batch * per
    for b in range(batch):
        rows[b] = list(rows[b]) + [free[taken + b]]
    lens = np.full(batch, cached + 1, dtype=np.int32)
    new = [(b, cached) for b in range(batch)]
    return Workload(f"llama70b-fp8-b{batch}-l{cached + 1}", seed, 64, 8, True, nb, lens,
                    _pad_tables(rows), new_tokens=new)


def llama70b_fp8_tp4(seed: int = 3) -> Workload:
    """One GPU's share of the 70B FP8 batch under 4-way tensor parallelism
    over KV heads ("Optimización de KV Cache ...", §5 serves the model on 4
    GPUs): the same 64 sequences and tables, 2 of the 8 KV heads and their 16
    query heads."""
    wl = llama70b_fp8(seed)
    wl.name = wl.name.replace("llama70b-fp8", "llama70b-fp8-tp4-share")
    wl.num_q_heads, wl.num_kv_heads = 16, 2
    return wl


def long_context(seed: int = 4, batch: int = 4, length: int = 131072,
                 partition_size: int = 512) -> Workload:
    """Batch 4 x 131072 tokens, FP8, split-KV into 512-token partitions; the
    pool holds exactly the sequences' blocks, shuffled."""
    rng = np.random.default_rng(seed)
    per = length // BS
    nb = batch * per
    perm = rng.permutation(nb).astype(np.int32).reshape(batch, per)
    lens = np.full(batch, length, dtype=np.int32)
    return Workload(f"long-fp8-b{batch}-l{length}", seed, 64, 8, True, nb, lens, perm,
                    partition_size=partition_size)


def shared_prefix(seed: int = 5, groups: int = 32, per_group: int = 8,
                  prefix_tokens: int = 2000, max_len: int = 32768) -> Workload:
    """256 sequences in groups of 8 sharing a 2000-token (125-block) prefix,
    then private tails; tail lengths log-normal (median 1024, sigma 1),
    clipped so 16 <= tail and 2000 + tail <= 32768.  FP8 KV, shuffled pool
    sized to 1.1x the blocks needed, rounded up to 1024."""
    rng = np.random.default_rng(seed)
    B = groups * per_group
    tails = np.clip(np.rint(np.exp(rng.normal(np.log(1024.0), 1.0, size=B))), 16,
                    max_len - prefix_tokens).astype(np.int64)
    pblocks = -(-prefix_tokens // BS)
    need = groups * pblocks + int(sum(-(-int(t) // BS) for t in tails))
    nb = int(-(-int(1.1 * need) // 1024) * 1024)
    free = list(rng.permutation(nb).astype(np.int32))
    rows, grp, pos = [], [], 0
    for g in range(groups):
        prefix = free[pos:pos + pblocks]
        pos += pblocks
        members = []
        for k in range(per_group):
            b = g * per_group + k
            n = -(-int(tails[b]) // BS)
            rows.append(list(prefix) + list(free[pos:pos + n]))
            pos += n
            members.append(b)
        grp.append(members)
    lens = (prefix_tokens + tails).astype(np.int32)
    return Workload(f"shared-prefix-fp8-b{B}", seed, 64, 8, True, nb, lens, _pad_tables(rows),
                    groups=grp, prefix_blocks=pblocks)


@dataclass
class PrefillWorkload:
    """A batch of prompt chunks: sequence b holds context_lens[b] tokens in
    the cache, the last chunk_lens[b] of which are the chunk's queries."""
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    fp8: bool
    num_blocks: int
    context_lens: np.ndarray            # int32 [B]
    chunk_lens: np.ndarray              # int32 [B]
    block_tables: np.ndarray            # int32 [B][max_blocks]

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def query_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.chunk_lens)]).astype(np.int32)

    @property
    def elem_bytes(self) -> int:
        return 1 if self.fp8 else 2

    def flops(self) -> int:
        """Algorithmic flops: for every chunk row at position p and query head,
        QK^T and PV over its p + 1 visible tokens, 2 * D flops each."""
        total = 0
        for L, n in zip(self.context_lens.astype(np.int64), self.chunk_lens.astype(np.int64)):
            first = L - n
            total += n * first + n * (n + 1) // 2     # sum over rows of (p + 1)
        return int(total) * self.num_q_heads * 4 * D


def _prefill(name, seed, lens, chunks, fp8=True):
    rng = np.random.default_rng(seed)
    nblk = [-(-int(L) // BS) for L in lens]
    nb = int(sum(nblk))
    perm = rng.permutation(nb).astype(np.int32)
    rows, pos = [], 0
    for n in nblk:
        rows.append(perm[pos:pos + n])
        pos += n
    return PrefillWorkload(name, seed, 64, 8, fp8, nb, np.asarray(lens, np.int32),
                           np.asarray(chunks, np.int32), _pad_tables(rows))


def prefill_128k(seed: int = 6) -> PrefillWorkload:
    """The last 8192-token chunk (the page's batched-token budget) of one
    131072-token prompt: 8192 query rows over 122880 earlier tokens plus the
    causal triangle; 70B layer shape, FP8 KV, shuffled pool."""
    return _prefill("prefill-fp8-b1-chunk8192-l131072", seed, [131072], [8192])


def prefill_mixed(seed: int = 7) -> PrefillWorkload:
    """Four prompts' chunks sharing an 8192-token budget (2048 each), at
    different depths: a first chunk, and chunks ending at 16K, 64K and 128K
    tokens; FP8 KV."""
    return _prefill("prefill-fp8-b4-chunk2048-mixed", seed, [2048, 16384, 65536, 131072],
                    [2048] * 4)


def prefill_128k_fp16(seed: int = 6) -> PrefillWorkload:
    """The 128K prompt's last 8192-token chunk with an fp16 cache."""
    return _prefill("prefill-fp16-b1-chunk8192-l131072", seed, [131072], [8192], fp8=False)


CONFIGS = {
    "tiny": tiny,
    "llama70b_fp16": llama70b_fp16,
    "llama70b_fp8": llama70b_fp8,
    "llama70b_fp8_tp4": llama70b_fp8_tp4,
    "long_context": long_context,
    "shared_prefix": shared_prefix,
}

PREFILL_CONFIGS = {
    "prefill_128k": prefill_128k,
    "prefill_mixed": prefill_mixed,
    "prefill_128k_fp16": prefill_128k_fp16,
}


def randn_f16(shape, seed: int, device: str = "cpu"):
    """N(0, 1) fp16 tensor drawn with a seeded torch generator on `device`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.float16, device=device)
    chunk = 1 << 26
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        out[i:i + m] = torch.randn(m, generator=g, device=device, dtype=torch.float32).half()
    return out.view(*shape)
