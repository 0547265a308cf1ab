"""GPU parity of the cascade decode over shared prefixes
(pkv_paged_attention_decode_cascade): each group's prefix blocks are attended
once for all its members, each tail on its own, and the partials merged.

Expected values come from the oracle only (its decode over the same bytes,
and its cache write of the newest rows for the writing variant): max abs
error 2e-3 with fp16 KV, 1e-2 with FP8 KV.  The pools after a writing call
must equal the oracle's write byte for byte.  Against the library's plain
decode the result agrees within the same bound (the split-KV identity; the
partials are summed in another order, so bits may differ).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import paged_kv_cache_270_amd as pkv  # noqa: E402
from paged_kv_cache_270_amd import workloads  # noqa: E402

from gpu_common import THREADS, TOL, Prepared, max_err  # noqa: E402

D = workloads.D


def _grouped(spec, solo, hq, hkv, fp8, seed):
    """Groups of sequences sharing a prefix, then sequences of their own.
    spec: list of (prefix_tokens, [tail lengths]) -- the prefix is whole
    blocks shared by every member, the tails start in fresh blocks; solo: the
    lengths of sequences in no group.  Returns the workload plus the groups
    and per-sequence prefix blocks a caller would pass."""
    rng = np.random.default_rng(seed)
    need = sum(-(-p // 16) + sum(-(-t // 16) for t in tails) for p, tails in spec)
    need += sum(-(-L // 16) for L in solo)
    nb = need + 8
    free = list(rng.permutation(nb).astype(np.int32))
    rows, lens, groups, prefix = [], [], [], []
    pos = 0
    for ptok, tails in spec:
        pb = -(-ptok // 16)
        pre = free[pos:pos + pb]
        pos += pb
        members = []
        for t in tails:
            n = -(-t // 16)
            rows.append(list(pre) + list(free[pos:pos + n]))
            pos += n
            members.append(len(lens))
            lens.append(pb * 16 + t)
            prefix.append(pb)
        groups.append(members)
    for L in solo:
        n = -(-L // 16)
        rows.append(list(free[pos:pos + n]))
        pos += n
        lens.append(L)
        prefix.append(0)
    width = max(1, max(len(r) for r in rows))
    tables = np.zeros((len(rows), width), dtype=np.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = r
    lens = np.asarray(lens, dtype=np.int32)
    new = [(b, int(L) - 1) for b, L in enumerate(lens) if L > 0]
    wl = workloads.Workload("cascade", seed, hq, hkv, fp8, nb, lens, tables, new_tokens=new)
    return wl, groups, np.asarray(prefix, dtype=np.int32)


def _group_array(groups, cap):
    """[n_groups][cap] member table, groups longer than cap split."""
    out = []
    for g in groups:
        for c in range(0, len(g), cap):
            part = g[c:c + cap]
            out.append(part + [-1] * (cap - len(part)))
    return np.asarray(out, dtype=np.int32).reshape(-1, cap)


def _cascade(prep, groups, prefix, cap, ps, write, name, order=None, tail_units=0,
             tail_map=None):
    wl = prep.wl
    B, Hkv, fp8 = wl.num_seqs, wl.num_kv_heads, wl.fp8
    garr = _group_array(groups, cap)
    d_groups = torch.from_numpy(garr).cuda()
    d_prefix = torch.from_numpy(prefix).cuda()
    key = val = None
    k_exp, v_exp = prep.k_host, prep.v_host
    if write:
        seqs = np.array([s for s, _ in wl.new_tokens], dtype=np.int64)
        key = torch.zeros((B, Hkv, D), dtype=torch.float16, device="cuda")
        val = torch.zeros_like(key)
        key[torch.from_numpy(seqs).cuda()] = prep.new_k
        val[torch.from_numpy(seqs).cuda()] = prep.new_v
        k_exp, v_exp = prep.k_host.copy(), prep.v_host.copy()
        oracle.reshape_and_cache(prep.new_k.cpu().numpy(), prep.new_v.cpu().numpy(), k_exp,
                                 v_exp, prep.new_slots_host, Hkv, fp8, prep.k_scale,
                                 prep.v_scale)
    ref = oracle.paged_attention_decode(prep.q_host, k_exp, v_exp, wl.block_tables,
                                        wl.context_lens, Hkv, fp8, prep.sm_scale, prep.k_scale,
                                        prep.v_scale, THREADS)
    out = torch.full(prep.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    pkv.pkv_paged_attention_decode_cascade(
        out, prep.q, key, val, prep.k_pool, prep.v_pool, prep.tables, prep.lens,
        wl.max_context_len, prep.layout, prep.sm_scale, d_prefix, d_groups,
        int(prefix.max()) if prefix.size else 0, prep.k_scale, prep.v_scale, ps,
        seq_order=None if order is None else torch.from_numpy(order).cuda(),
        tail_units=tail_units,
        tail_map=None if tail_map is None else torch.from_numpy(tail_map).cuda())
    torch.cuda.synchronize()
    if write:
        assert np.array_equal(prep.k_pool.cpu().numpy(), k_exp)
        assert np.array_equal(prep.v_pool.cpu().numpy(), v_exp)
    got = out.cpu().numpy()
    err = max_err(got, ref)
    print(f"[parity] cascade {name} P={ps} write={write}: max abs err {err:.3e} "
          f"(tol {TOL[fp8]:.0e})", flush=True)
    assert np.isfinite(got).all()
    assert err <= TOL[fp8]
    return got


# groups of 1, 2, 3 and 9 members (9 > cap 8: split in two), prefixes of 1 to
# 70 blocks, tails of 1 token to several partitions; a member whose length is
# exactly its prefix is not allowed (16 * S < L), so tails are >= 1
SPEC = [(16, [1]), (32, [1, 17]), (1120, [5, 300, 2000]),
        (208, [16, 15, 33, 64, 1, 700, 129, 2, 999])]
SOLO = [0, 1, 37, 1500]


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("ps", [0, 16, 64, 512])
@pytest.mark.parametrize("write", [False, True])
def test_cascade_matches_oracle(fp8, ps, write):
    wl, groups, prefix = _grouped(SPEC, SOLO, 8, 2, fp8, seed=71 + ps)
    prep = Prepared(wl)
    _cascade(prep, groups, prefix, 8, ps, write, f"fp8={fp8}")


@pytest.mark.parametrize("fp8", [False, True])
def test_cascade_tail_order(fp8):
    """Tails scheduled in a given order (longest first, and reversed) give
    the same results as batch order."""
    wl, groups, prefix = _grouped(SPEC, SOLO, 8, 2, fp8, seed=77)
    prep = Prepared(wl)
    tail = wl.context_lens.astype(np.int64) - 16 * prefix
    order = np.argsort(-tail, kind="stable").astype(np.int32)
    a = _cascade(prep, groups, prefix, 8, 0, False, "longest tail first", order)
    b = _cascade(prep, groups, prefix, 8, 0, False, "reversed", order[::-1].copy())
    c = _cascade(prep, groups, prefix, 8, 0, False, "batch order")
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))
    assert np.array_equal(b.view(np.uint32), c.view(np.uint32))


def test_cascade_order_skips_entries_out_of_range():
    """An order entry outside the batch is skipped; every listed sequence is
    still correct (the one not listed has unspecified output)."""
    wl, groups, prefix = _grouped([], [100, 300, 50], 8, 2, True, seed=78)
    prep = Prepared(wl)
    out = torch.full(prep.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    order = torch.tensor([2, 99, 0], dtype=torch.int32, device="cuda")
    pkv.pkv_paged_attention_decode_cascade(
        out, prep.q, None, None, prep.k_pool, prep.v_pool, prep.tables, prep.lens,
        wl.max_context_len, prep.layout, prep.sm_scale, None, None, 0, prep.k_scale,
        prep.v_scale, 0, seq_order=order)
    got = out.cpu().numpy()
    ref = prep.oracle_decode()
    assert max_err(got[[0, 2]], ref[[0, 2]]) <= TOL[True]


@pytest.mark.parametrize("hq,hkv", [(16, 1), (4, 4), (6, 2), (32, 2)])
def test_cascade_group_sizes(hq, hkv):
    """16 / G members per wave: 1 (G = 16), 4 (G = 1), 5 (G = 3: one column
    left over), 1 (G = 16 at two KV heads)."""
    wl, groups, prefix = _grouped(SPEC, SOLO, hq, hkv, True, seed=72 + hq)
    prep = Prepared(wl)
    _cascade(prep, groups, prefix, 8, 0, True, f"Hq={hq} Hkv={hkv}")


@pytest.mark.parametrize("cap", [1, 3, 16])
def test_cascade_group_cap(cap):
    wl, groups, prefix = _grouped(SPEC, SOLO, 8, 2, True, seed=73)
    prep = Prepared(wl)
    _cascade(prep, groups, prefix, cap, 0, False, f"cap={cap}")


def test_cascade_without_groups_equals_plain_decode():
    """No groups: every sequence is decoded on its own, as by the plain call."""
    wl, _, _ = _grouped([], [1, 37, 1500, 0, 4096], 8, 2, True, seed=74)
    prep = Prepared(wl)
    out = torch.empty(prep.q.shape, dtype=torch.float32, device="cuda")
    pkv.pkv_paged_attention_decode_cascade(
        out, prep.q, None, None, prep.k_pool, prep.v_pool, prep.tables, prep.lens,
        wl.max_context_len, prep.layout, prep.sm_scale, None, None, 0, prep.k_scale,
        prep.v_scale, 0)
    plain = prep.gpu_decode(partition_size=0)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), plain.view(np.uint32))


def test_cascade_from_pool_forks():
    """Groups found by the host pool from forked sequences: the cascade step
    (write + decode) leaves the pools as the plain step does and matches the
    oracle."""
    fp8, Hkv, Hq = True, 2, 8
    rng = np.random.default_rng(75)
    NB = 512
    pool = pkv.BlockPool(NB, shuffle_seed=75)
    seqs = []
    for plen, n in ((500, 4), (333, 3), (64, 2)):
        root = pool.create()
        pool.append(root, plen)
        fam = [root] + [pool.fork(root) for _ in range(n - 1)]
        for s in fam:  # private tails, the last token being the one decoded
            pool.append(s, int(rng.integers(1, 400)))
        seqs += fam
    solo = pool.create()
    pool.append(solo, 77)
    seqs.append(solo)
    lens = np.array([pool.seq_len(s) for s in seqs], dtype=np.int32)
    rows = [pool.block_table(s) for s in seqs]
    tables = np.zeros((len(seqs), max(len(r) for r in rows)), dtype=np.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = r
    prefix, garr, max_pre, order = pool.prefix_groups(seqs, 8, with_order=True)
    assert garr.shape[0] == 3 and max_pre == 31       # 500 tokens: 31 whole blocks
    new = [(b, int(L) - 1) for b, L in enumerate(lens)]
    wl = workloads.Workload("cascade-pool", 75, Hq, Hkv, fp8, NB, lens, tables, new_tokens=new)
    prep = Prepared(wl)
    groups = [[int(m) for m in g if m >= 0] for g in garr]
    _cascade(prep, groups, prefix, 8, 0, True, "pool forks", order)


def _pool_built(wl):
    """The workload's sequences grown in the library's host block pool as
    the benchmark grows them: each group's leader takes the prefix, the
    other members fork it, every member appends its tail, then one call
    assigns every sequence's newest token.  Returns the tables, lengths,
    prefix groups and the longest-tail-first order the pool reports."""
    pool = pkv.BlockPool(wl.num_blocks, shuffle_seed=wl.seed)
    lens = [int(x) for x in wl.context_lens]
    seqs = []
    for members in wl.groups:
        leader = pool.create()
        pool.append(leader, wl.prefix_blocks * 16)
        ids = [leader] + [pool.fork(leader) for _ in members[1:]]
        for sid, b in zip(ids, members):
            pool.append(sid, lens[b] - wl.prefix_blocks * 16 - 1)
            seqs.append(sid)
    pool.append_each(seqs)
    got = np.array([pool.seq_len(s) for s in seqs], dtype=np.int32)
    assert np.array_equal(got, wl.context_lens)
    rows = [pool.block_table(s) for s in seqs]
    tables = np.zeros((len(seqs), max(len(r) for r in rows)), dtype=np.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = r
    prefix, garr, max_pre, order = pool.prefix_groups(seqs, 8, with_order=True)
    P = pkv.pkv_decode_partition_size(len(seqs), wl.num_kv_heads, int(got.max()),
                                      pkv.PKV_FP8_E4M3FN, 0)
    units = pool.cascade_tail_units(seqs, prefix, max_pre, P)
    tmap = pool.cascade_tail_map(seqs, prefix, max_pre, P, order)
    assert len(tmap) == units
    return tables, got, prefix, garr, max_pre, order, units, tmap


def test_cascade_shared_prefix_full_step():
    """The 256-sequence shared-prefix batch at full size (FP8, 32 groups of 8
    with a 125-block prefix), run as the benchmark's step runs it: sequences
    grown in the host pool, groups, the longest-tail order and the list of
    tail units from the pool, the automatic partition size, and each
    sequence's newest K/V rows written by the cascade call itself.  Both
    pools must equal the oracle's write byte for byte, and all 256 outputs
    must match the oracle's decode."""
    base = workloads.shared_prefix()
    tables, lens, prefix, garr, max_pre, order, units, tmap = _pool_built(base)
    assert garr.shape[0] == 32 and max_pre == base.prefix_blocks
    B = base.num_seqs
    new = [(b, int(L) - 1) for b, L in enumerate(lens)]
    wl = workloads.Workload(base.name, base.seed, base.num_q_heads, base.num_kv_heads, True,
                            base.num_blocks, lens, tables, new_tokens=new)
    prep = Prepared(wl)
    groups = [[int(m) for m in g if m >= 0] for g in garr]
    assert sorted(m for g in groups for m in g) == list(range(B))
    got = _cascade(prep, groups, prefix, 8, 0, True, "shared-prefix B=256 full step", order,
                   tail_units=units, tail_map=tmap)
    assert got.shape == (B, wl.num_q_heads, D)


def test_cascade_block_scales_shared_prefix_full():
    """The 256-sequence shared-prefix batch at full size over per-(block, KV
    head) FP8 scales, decoded as the benchmark's block-scale step decodes it
    (groups, longest-tail order and tail units from the host pool, the
    automatic partition size; the prefix items' four waves share each tile).
    Every slot of the pool is written by the oracle's dynamic write from rows
    whose magnitude varies from slot to slot, so the scales differ from block
    to block and the waves' V reference grows; all 256 outputs must match the
    oracle's decode with block scales."""
    base = workloads.shared_prefix()
    tables, lens, prefix, garr, max_pre, order, units, tmap = _pool_built(base)
    B, Hq, Hkv, NB = base.num_seqs, base.num_q_heads, base.num_kv_heads, base.num_blocks
    T = NB * 16
    mag = torch.exp(1.5 * torch.randn((T, 1, 1), generator=torch.Generator().manual_seed(83)))
    mag = mag.cuda()
    k = (workloads.randn_f16((T, Hkv, D), 84, "cuda").float() * mag).half().cpu().numpy()
    v = (workloads.randn_f16((T, Hkv, D), 85, "cuda").float() * mag.flip(0)).half().cpu().numpy()
    torch.cuda.empty_cache()
    n = NB * Hkv * 16 * D
    kh, vh = np.zeros(n, np.uint8), np.zeros(n, np.uint8)
    ksh, vsh = np.zeros((NB, Hkv), np.float32), np.zeros((NB, Hkv), np.float32)
    oracle.reshape_and_cache_dynamic(k, v, kh, vh, ksh, vsh, np.arange(T, dtype=np.int64), Hkv)
    del k, v
    layout = pkv.CacheLayout(NB, Hkv, pkv.PKV_FP8_E4M3FN)
    q = workloads.randn_f16((B, Hq, D), 86, "cuda")
    sm = float(np.float32(1 / np.sqrt(D)))
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    pkv.pkv_paged_attention_decode_cascade_dynamic(
        out, q, torch.from_numpy(kh).cuda(), torch.from_numpy(vh).cuda(),
        torch.from_numpy(ksh).cuda(), torch.from_numpy(vsh).cuda(),
        torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(), int(lens.max()),
        layout, sm, torch.from_numpy(prefix).cuda(), torch.from_numpy(garr).cuda(), max_pre, 0,
        seq_order=torch.from_numpy(order).cuda(), tail_units=units,
        tail_map=torch.from_numpy(tmap).cuda())
    torch.cuda.synchronize()
    ref = oracle.paged_attention_decode_dynamic(q.cpu().numpy(), kh, vh, ksh, vsh, tables, lens,
                                                Hkv, sm, THREADS)
    got = out.cpu().numpy()
    err = max_err(got, ref)
    print(f"[parity] cascade block scales, shared-prefix B=256 full: max abs err {err:.3e}",
          flush=True)
    assert np.isfinite(got).all()
    assert err <= TOL[True]


def test_cascade_rejects_bad_arguments():
    wl, groups, prefix = _grouped(SPEC, SOLO, 8, 2, True, seed=76)
    prep = Prepared(wl)
    out = torch.empty(prep.q.shape, dtype=torch.float32, device="cuda")
    key = torch.zeros((wl.num_seqs, 2, D), dtype=torch.float16, device="cuda")
    garr = torch.from_numpy(_group_array(groups, 8)).cuda()
    pre = torch.from_numpy(prefix).cuda()
    L = pkv.load_library()
    lay = prep.layout
    import ctypes
    # key without value
    st = L.pkv_paged_attention_decode_cascade(
        out.data_ptr(), prep.q.data_ptr(), key.data_ptr(), None, prep.k_pool.data_ptr(),
        prep.v_pool.data_ptr(), prep.tables.data_ptr(), prep.tables.shape[1],
        prep.lens.data_ptr(), None, pre.data_ptr(), garr.data_ptr(), garr.shape[0], 8,
        int(prefix.max()), None, 0, None, wl.num_seqs, 8, wl.max_context_len, ctypes.byref(lay),
        prep.sm_scale, prep.k_scale, prep.v_scale, 0, None, 0, None)
    assert st == pkv.PKV_ERR_INVALID_ARG
    # workspace smaller than the cascade needs (the plain size is smaller)
    plain = pkv.pkv_decode_workspace_bytes(wl.num_seqs, 8, 2, wl.max_context_len,
                                           lay.dtype, 64)
    need = pkv.pkv_decode_cascade_workspace_bytes(wl.num_seqs, 8, 2, wl.max_context_len,
                                                  int(prefix.max()), lay.dtype, 64)
    assert need > plain
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    st = L.pkv_paged_attention_decode_cascade(
        out.data_ptr(), prep.q.data_ptr(), None, None, prep.k_pool.data_ptr(),
        prep.v_pool.data_ptr(), prep.tables.data_ptr(), prep.tables.shape[1],
        prep.lens.data_ptr(), None, pre.data_ptr(), garr.data_ptr(), garr.shape[0], 8,
        int(prefix.max()), None, 0, None, wl.num_seqs, 8, wl.max_context_len, ctypes.byref(lay),
        prep.sm_scale, prep.k_scale, prep.v_scale, 64, ws.data_ptr(), ws.numel(), None)
    assert st == pkv.PKV_ERR_WORKSPACE
    # more items plus sequences than one grid dimension holds (G = 4: one item
    # per group of 4; 65535 items + the sequences > 65535), with a workspace
    # large enough, so the count alone is rejected -- before any launch
    big = torch.empty(pkv.pkv_decode_cascade_workspace_bytes(
        wl.num_seqs, 8, 2, wl.max_context_len, int(prefix.max()), lay.dtype, 64),
        dtype=torch.uint8, device="cuda")
    st = L.pkv_paged_attention_decode_cascade(
        out.data_ptr(), prep.q.data_ptr(), None, None, prep.k_pool.data_ptr(),
        prep.v_pool.data_ptr(), prep.tables.data_ptr(), prep.tables.shape[1],
        prep.lens.data_ptr(), None, pre.data_ptr(), garr.data_ptr(), 65535, 4,
        int(prefix.max()), None, 0, None, wl.num_seqs, 8, wl.max_context_len, ctypes.byref(lay),
        prep.sm_scale, prep.k_scale, prep.v_scale, 64, big.data_ptr(), big.numel(), None)
    assert st == pkv.PKV_ERR_INVALID_ARG


@pytest.mark.parametrize("ps", [0, 16, 512])
def test_cascade_block_scales_matches_oracle(ps):
    """Per-(block, KV head) FP8 scales: every slot of every block written by
    the oracle's dynamic write from rows of varying magnitude (so scales
    differ from block to block), then the cascade against the oracle's
    decode with block scales."""
    wl, groups, prefix = _grouped(SPEC, SOLO, 8, 2, True, seed=79 + ps)
    NB, Hkv = wl.num_blocks, wl.num_kv_heads
    rng = np.random.default_rng(80 + ps)
    T = NB * 16
    mag = np.exp(1.5 * rng.standard_normal((T, 1, 1)))
    k = (rng.standard_normal((T, Hkv, D)) * mag).astype(np.float16)
    v = (rng.standard_normal((T, Hkv, D)) * mag[::-1]).astype(np.float16)
    n = NB * Hkv * 16 * D
    kh, vh = np.zeros(n, np.uint8), np.zeros(n, np.uint8)
    ksh, vsh = np.zeros((NB, Hkv), np.float32), np.zeros((NB, Hkv), np.float32)
    oracle.reshape_and_cache_dynamic(k, v, kh, vh, ksh, vsh, np.arange(T, dtype=np.int64), Hkv)
    layout = pkv.CacheLayout(NB, Hkv, pkv.PKV_FP8_E4M3FN)
    q = workloads.randn_f16((wl.num_seqs, 8, D), 81 + ps, "cuda")
    sm = float(np.float32(1 / np.sqrt(D)))
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    tail = wl.context_lens.astype(np.int64) - 16 * prefix
    order = np.argsort(-tail, kind="stable").astype(np.int32)
    pkv.pkv_paged_attention_decode_cascade_dynamic(
        out, q, torch.from_numpy(kh).cuda(), torch.from_numpy(vh).cuda(),
        torch.from_numpy(ksh).cuda(), torch.from_numpy(vsh).cuda(),
        torch.from_numpy(wl.block_tables).cuda(), torch.from_numpy(wl.context_lens).cuda(),
        wl.max_context_len, layout, sm, torch.from_numpy(prefix).cuda(),
        torch.from_numpy(_group_array(groups, 8)).cuda(), int(prefix.max()), ps,
        seq_order=torch.from_numpy(order).cuda())
    torch.cuda.synchronize()
    ref = oracle.paged_attention_decode_dynamic(q.cpu().numpy(), kh, vh, ksh, vsh,
                                                wl.block_tables, wl.context_lens, Hkv, sm,
                                                THREADS)
    got = out.cpu().numpy()
    err = max_err(got, ref)
    print(f"[parity] cascade block scales P={ps}: max abs err {err:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err <= TOL[True]


@pytest.mark.parametrize("seed", range(6))
def test_cascade_random_groups(seed):
    """Random batches: 1 to 6 groups of 1 to 10 members with prefixes of 1 to
    40 blocks and tails of 1 to 600 tokens, sequences in no group, random
    head groupings, fp16 or FP8, random split sizes, groups in random slots
    of a padded group table, tails in a random order; against the oracle."""
    rng = np.random.default_rng(900 + seed)
    spec = [(16 * int(rng.integers(1, 41)), [int(t) for t in rng.integers(1, 601,
                                                                          rng.integers(1, 11))])
            for _ in range(int(rng.integers(1, 7)))]
    solo = [int(x) for x in rng.integers(0, 900, int(rng.integers(0, 6)))]
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 8, 16]))
    fp8 = bool(seed % 2)
    wl, groups, prefix = _grouped(spec, solo, g * hkv, hkv, fp8, seed=910 + seed)
    cap = int(rng.integers(max(len(m) for m in groups), 13))
    garr = _group_array(groups, cap)
    # groups in random rows, among rows of empty slots (skipped items)
    rows = np.full((garr.shape[0] + 2, cap), -1, dtype=np.int32)
    rows[rng.permutation(rows.shape[0])[:garr.shape[0]]] = garr
    prep = Prepared(wl)
    order = rng.permutation(wl.num_seqs).astype(np.int32)
    ps = int(rng.choice([0, 16, 48, 256]))
    out = torch.full(prep.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    pkv.pkv_paged_attention_decode_cascade(
        out, prep.q, None, None, prep.k_pool, prep.v_pool, prep.tables, prep.lens,
        wl.max_context_len, prep.layout, prep.sm_scale, torch.from_numpy(prefix).cuda(),
        torch.from_numpy(rows).cuda(), int(prefix.max()), prep.k_scale, prep.v_scale, ps,
        seq_order=torch.from_numpy(order).cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    err = max_err(got, prep.oracle_decode())
    print(f"[parity] cascade random seed={seed} G={g} Hkv={hkv} fp8={fp8} P={ps}: "
          f"max abs err {err:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err <= TOL[fp8]


def test_cascade_batch_above_the_flat_grid():
    """2100 short sequences (groups of 8 over 1- or 2-block prefixes, and
    sequences in no group): more than the flat grid's batch limit, so the
    (partition, KV head, item or sequence) grid runs; against the oracle."""
    rng = np.random.default_rng(95)
    spec = [(16 * int(rng.integers(1, 3)), [int(t) for t in rng.integers(1, 40, 8)])
            for _ in range(250)]
    solo = [int(x) for x in rng.integers(0, 60, 100)]
    wl, groups, prefix = _grouped(spec, solo, 8, 2, True, seed=96)
    assert wl.num_seqs == 2100
    prep = Prepared(wl)
    tail = wl.context_lens.astype(np.int64) - 16 * prefix
    order = np.argsort(-tail, kind="stable").astype(np.int32)
    _cascade(prep, groups, prefix, 8, 0, True, "B=2100", order)


def test_cascade_tail_units_change_no_result():
    """The launch sized by the exact tail count, by an underestimate (each
    workgroup then takes several units), by an overestimate and by the
    default bound: the same outputs bit for bit, and the oracle's."""
    rng = np.random.default_rng(97)
    spec = [(16 * int(rng.integers(1, 30)), [int(t) for t in rng.integers(1, 900, 6)])
            for _ in range(5)]
    solo = [0, 5, 1200]
    wl, groups, prefix = _grouped(spec, solo, 8, 2, True, seed=98)
    prep = Prepared(wl)
    tail = wl.context_lens.astype(np.int64) - 16 * prefix
    order = np.argsort(-tail, kind="stable").astype(np.int32)
    ps = 64
    nblk = -(-wl.context_lens.astype(np.int64) // 16) - prefix
    exact = int(np.maximum(1, -(-nblk // (ps // 16))).sum())
    outs = []
    for tu in (exact, 1, 3, exact + 40, 0):
        outs.append(_cascade(prep, groups, prefix, 8, ps, False, f"tail_units={tu}", order,
                             tail_units=tu))
    # the same units listed by a map, and the map with entries outside the
    # batch (skipped) mixed in
    per = ps // 16
    tmap = np.array([(b, u) for b in order for u in range(max(1, -(-int(nblk[b]) // per)))],
                    dtype=np.int32)
    assert len(tmap) == exact
    outs.append(_cascade(prep, groups, prefix, 8, ps, False, "tail map", order,
                         tail_units=exact, tail_map=tmap))
    junk = np.array([(-1, 0), (wl.num_seqs, 0), (0, -1)], dtype=np.int32)
    mixed = np.concatenate([tmap[:5], junk, tmap[5:]])
    outs.append(_cascade(prep, groups, prefix, 8, ps, False, "tail map with junk", order,
                         tail_units=len(mixed), tail_map=mixed))
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
