"""Pins of the oracle's cache write, layout and decode attention.

Decode attention over a paged cache must equal ordinary scaled-dot-product
attention over the same tokens taken in logical order, whatever physical
blocks hold them ("LLM Primer VI, Capítulo 8 — Gestión de caché KV", §8.1:
the kernel gathers keys and values through the block table instead of slicing
a contiguous slab).  The pins below compare the oracle with a library
attention (torch, fp64, CPU), with closed forms, and with invariances that a
dropped term, a wrong index or a swapped operand would break.
"""
import math

import numpy as np
import pytest
import torch

from conftest import golden

BS, D = 16, 128


def _tables_from_perm(rng, lens, num_blocks):
    """Random physical placement: blocks handed out from a shuffled pool."""
    nblk = [-(-int(L) // BS) for L in lens]
    maxb = max(1, max(nblk))
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = np.zeros((len(lens), maxb), dtype=np.int32)
    pos = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[pos:pos + n]
        # entries past the sequence's blocks hold ids of other blocks (ignored)
        bt[b, n:] = perm[(pos + n) % num_blocks]
        pos += n
    return bt


def _write_sequences(orc, rng, lens, Hkv, fp8, num_blocks, k_scale=1.0, v_scale=1.0, bt=None,
                     fill_garbage=True):
    """Build logical K/V (fp16, N(0,1)), store them through the oracle write."""
    e = 1 if fp8 else 2
    if bt is None:
        bt = _tables_from_perm(rng, lens, num_blocks)
    nbytes = num_blocks * Hkv * BS * D * e
    if fill_garbage:
        k_pool = rng.integers(0, 256, nbytes, dtype=np.uint8)
        v_pool = rng.integers(0, 256, nbytes, dtype=np.uint8)
        if fp8:  # keep garbage finite so a leaked masked slot would show as a wrong value, not NaN
            k_pool[(k_pool & 0x7F) == 0x7F] = 0x10
            v_pool[(v_pool & 0x7F) == 0x7F] = 0x10
        else:
            k_pool = rng.standard_normal(nbytes // 2).astype(np.float16).view(np.uint8).copy()
            v_pool = rng.standard_normal(nbytes // 2).astype(np.float16).view(np.uint8).copy()
    else:
        k_pool = np.zeros(nbytes, dtype=np.uint8)
        v_pool = np.zeros(nbytes, dtype=np.uint8)
    Ks, Vs = [], []
    for b, L in enumerate(lens):
        k = rng.standard_normal((L, Hkv, D)).astype(np.float16)
        v = rng.standard_normal((L, Hkv, D)).astype(np.float16)
        slots = orc.slots_for(bt, [b] * L, range(L))
        orc.reshape_and_cache(k, v, k_pool, v_pool, slots, Hkv, fp8, k_scale, v_scale)
        Ks.append(k)
        Vs.append(v)
    return k_pool, v_pool, bt, Ks, Vs


def _dequant(x16, scale, fp8):
    """Value the cache holds for fp16 input x16: itself (fp16 pool) or the
    library's E4M3 cast of x/scale times scale (FP8 pool)."""
    x = torch.from_numpy(x16.astype(np.float32))
    if not fp8:
        return x.double()
    u = x / torch.tensor(np.float32(scale))
    return u.to(torch.float8_e4m3fn).to(torch.float64) * float(np.float32(scale))


def _sdpa_reference(q, Ks, Vs, Hkv, sm_scale, fp8, k_scale, v_scale):
    """Library attention (torch SDPA, fp64 CPU) over logically ordered rows,
    with each KV head repeated for its G query heads."""
    B, Hq, _ = q.shape
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        if Ks[b].shape[0] == 0:
            continue
        k = _dequant(Ks[b], k_scale, fp8).permute(1, 0, 2).repeat_interleave(G, dim=0)
        v = _dequant(Vs[b], v_scale, fp8).permute(1, 0, 2).repeat_interleave(G, dim=0)
        qq = torch.from_numpy(q[b].astype(np.float64)).unsqueeze(1)
        o = torch.nn.functional.scaled_dot_product_attention(
            qq.unsqueeze(0), k.unsqueeze(0).contiguous(), v.unsqueeze(0).contiguous(),
            scale=float(np.float32(sm_scale)))
        out[b] = o[0, :, 0, :].numpy()
    return out


# ------------------------------------------------------------------ layout

def test_layout_offsets_golden(orc):
    table = golden("cache_layout.txt")
    assert len(table) >= 20
    for key, val in table.items():
        kind, e, t, d = key.split()
        fn = orc.k_offset if kind == "K" else orc.v_offset
        assert fn(int(t), int(d), int(e)) == int(val), key


@pytest.mark.parametrize("e", [1, 2])
def test_layout_is_a_bijection_on_the_tile(orc, e):
    for fn in (orc.k_offset, orc.v_offset):
        offs = sorted(fn(t, d, e) for t in range(BS) for d in range(D))
        assert offs == list(range(BS * D))


def test_slot_follows_block_table_figure(orc):
    g = golden("block_table_figure.txt")
    row = [int(x) for x in g["table_req_a"].split()]
    for tok in (0, 20, 40, 47):
        assert orc.slot(row, tok) == int(g[f"token_{tok}_slot"])


# ------------------------------------------------------------------- write

@pytest.mark.parametrize("fp8", [False, True])
def test_write_places_bytes_at_documented_offsets(orc, fp8):
    rng = np.random.default_rng(11)
    Hkv, NB, e = 2, 6, (1 if fp8 else 2)
    key = rng.standard_normal((5, Hkv, D)).astype(np.float16)
    val = rng.standard_normal((5, Hkv, D)).astype(np.float16)
    slots = np.array([3, 17, -1, 95, 40], dtype=np.int64)
    ks, vs = np.float32(0.01), np.float32(0.02)
    kp = np.full(NB * Hkv * BS * D * e, 0xA5, dtype=np.uint8)
    vp = kp.copy()
    orc.reshape_and_cache(key, val, kp, vp, slots, Hkv, fp8, ks, vs)
    expect_k = np.full_like(kp, 0xA5)
    expect_v = expect_k.copy()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        blk, t = divmod(int(s), BS)
        for h in range(Hkv):
            base = (blk * Hkv + h) * BS * D
            for d in range(D):
                ka = (base + orc.k_offset(t, d, e)) * e
                va = (base + orc.v_offset(t, d, e)) * e
                if fp8:
                    # library cast of the correctly rounded fp32 quotient
                    expect_k[ka] = torch.tensor(np.float32(key[i, h, d]) / ks).to(
                        torch.float8_e4m3fn).view(torch.uint8).item()
                    expect_v[va] = torch.tensor(np.float32(val[i, h, d]) / vs).to(
                        torch.float8_e4m3fn).view(torch.uint8).item()
                else:
                    expect_k[ka:ka + 2] = key[i, h, d:d + 1].view(np.uint8)
                    expect_v[va:va + 2] = val[i, h, d:d + 1].view(np.uint8)
    assert np.array_equal(kp, expect_k)
    assert np.array_equal(vp, expect_v)


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (16, 1), (6, 3)])
def test_decode_matches_library_sdpa(orc, fp8, Hq, Hkv):
    rng = np.random.default_rng(100 + Hq * 7 + Hkv + int(fp8))
    lens = [1, 5, 16, 17, 33, 70]
    ks, vs = (np.float32(0.011), np.float32(0.013)) if fp8 else (1.0, 1.0)
    kp, vp, bt, Ks, Vs = _write_sequences(orc, rng, lens, Hkv, fp8, 64, ks, vs)
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float16)
    sm = np.float32(1 / math.sqrt(D))
    got = orc.paged_attention_decode(q, kp, vp, bt, lens, Hkv, fp8, sm, ks, vs)
    ref = _sdpa_reference(q, Ks, Vs, Hkv, sm, fp8, ks, vs)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_decode_zero_length_gives_zeros(orc):
    rng = np.random.default_rng(5)
    lens = [0, 3]
    kp, vp, bt, _, _ = _write_sequences(orc, rng, lens, 2, False, 8)
    q = rng.standard_normal((2, 4, D)).astype(np.float16)
    out = orc.paged_attention_decode(q, kp, vp, bt, lens, 2, False, 0.1)
    assert np.all(out[0] == 0.0)
    assert np.all(np.isfinite(out[1]))


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_single_token_returns_its_value_row(orc, fp8):
    rng = np.random.default_rng(6)
    vs = np.float32(0.037) if fp8 else 1.0
    kp, vp, bt, Ks, Vs = _write_sequences(orc, rng, [1, 1], 2, fp8, 8, 0.05, vs)
    q = rng.standard_normal((2, 4, D)).astype(np.float16)
    out = orc.paged_attention_decode(q, kp, vp, bt, [1, 1], 2, fp8, 0.3, 0.05, vs)
    for b in range(2):
        for h in range(4):
            expect = _dequant(Vs[b][0, h // 2], vs, fp8).numpy()
            assert np.array_equal(out[b, h], expect)


def test_decode_zero_query_is_mean_of_values(orc):
    rng = np.random.default_rng(8)
    lens = [37, 64]
    kp, vp, bt, Ks, Vs = _write_sequences(orc, rng, lens, 2, False, 16)
    q = np.zeros((2, 4, D), dtype=np.float16)
    out = orc.paged_attention_decode(q, kp, vp, bt, lens, 2, False, 0.2)
    for b in range(2):
        for h in range(4):
            mean = Vs[b][:, h // 2].astype(np.float64).mean(axis=0)
            assert np.max(np.abs(out[b, h] - mean)) < 1e-13


def test_decode_two_tokens_closed_form(orc):
    """q = e_0 * a, k_0 = e_0 * 1, k_1 = 0: logits differ by sm*a, so the
    output is sigmoid(sm*a) v_0 + sigmoid(-sm*a) v_1."""
    Hkv, NB = 1, 4
    kp = np.zeros(NB * Hkv * BS * D * 2, dtype=np.uint8)
    vp = kp.copy()
    rng = np.random.default_rng(9)
    k = np.zeros((2, 1, D), dtype=np.float16)
    k[0, 0, 0] = 1.0
    v = rng.standard_normal((2, 1, D)).astype(np.float16)
    bt = np.array([[3]], dtype=np.int32)
    orc.reshape_and_cache(k, v, kp, vp, np.array([48, 49]), Hkv, False)
    a, sm = 3.0, np.float32(0.5)
    q = np.zeros((1, 1, D), dtype=np.float16)
    q[0, 0, 0] = a
    out = orc.paged_attention_decode(q, kp, vp, bt, [2], Hkv, False, sm)
    z = float(sm) * a
    w0 = 1 / (1 + math.exp(-z))
    expect = w0 * v[0, 0].astype(np.float64) + (1 - w0) * v[1, 0].astype(np.float64)
    assert np.max(np.abs(out[0, 0] - expect)) < 1e-14


def test_decode_huge_gap_selects_one_row(orc):
    Hkv, NB = 1, 4
    kp = np.zeros(NB * BS * D * 2, dtype=np.uint8)
    vp = kp.copy()
    rng = np.random.default_rng(10)
    k = np.zeros((20, 1, D), dtype=np.float16)
    k[13, 0, :] = 1.0
    v = rng.standard_normal((20, 1, D)).astype(np.float16)
    bt = np.array([[2, 0]], dtype=np.int32)
    orc.reshape_and_cache(k, v, kp, vp, orc.slots_for(bt, [0] * 20, range(20)), Hkv, False)
    q = np.full((1, 1, D), 8.0, dtype=np.float16)
    out = orc.paged_attention_decode(q, kp, vp, bt, [20], Hkv, False, 1.0)
    assert np.max(np.abs(out[0, 0] - v[13, 0].astype(np.float64))) < 1e-300 + 1e-12


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_is_invariant_under_block_permutation(orc, fp8):
    """Move every physical block to a new id and rewrite the tables to
    match: the output must not change by a single bit."""
    rng = np.random.default_rng(12)
    lens = [70, 3, 129]
    Hkv, NB, e = 2, 32, (1 if fp8 else 2)
    kp, vp, bt, _, _ = _write_sequences(orc, rng, lens, Hkv, fp8, NB, 0.02, 0.03)
    q = rng.standard_normal((3, 8, D)).astype(np.float16)
    out1 = orc.paged_attention_decode(q, kp, vp, bt, lens, Hkv, fp8, 0.09, 0.02, 0.03)
    perm = rng.permutation(NB)
    tile = Hkv * BS * D * e
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    for old in range(NB):
        new = perm[old]
        kp2[new * tile:(new + 1) * tile] = kp[old * tile:(old + 1) * tile]
        vp2[new * tile:(new + 1) * tile] = vp[old * tile:(old + 1) * tile]
    bt2 = perm[bt].astype(np.int32)
    out2 = orc.paged_attention_decode(q, kp2, vp2, bt2, lens, Hkv, fp8, 0.09, 0.02, 0.03)
    assert np.array_equal(out1, out2)


def test_decode_shared_prefix_equals_copied_prefix(orc):
    """Two sequences reading one shared prefix block set give bit-identical
    results to the same sequences holding private copies of it."""
    rng = np.random.default_rng(13)
    Hkv, NB, e = 1, 16, 1
    tile = Hkv * BS * D * e
    kp = rng.integers(0, 0x70, NB * tile, dtype=np.uint8)
    vp = rng.integers(0, 0x70, NB * tile, dtype=np.uint8)
    # shared: both sequences use blocks 0,1 as prefix, then private tails 2 / 3
    shared = np.array([[0, 1, 2], [0, 1, 3]], dtype=np.int32)
    # copied: sequence 1's prefix lives in blocks 4,5 (byte copies of 0,1)
    kp[4 * tile:6 * tile] = kp[0:2 * tile]
    vp[4 * tile:6 * tile] = vp[0:2 * tile]
    copied = np.array([[0, 1, 2], [4, 5, 3]], dtype=np.int32)
    q = rng.standard_normal((2, 4, D)).astype(np.float16)
    lens = [40, 45]
    a = orc.paged_attention_decode(q, kp, vp, shared, lens, Hkv, True, 0.08, 0.05, 0.07)
    b = orc.paged_attention_decode(q, kp, vp, copied, lens, Hkv, True, 0.08, 0.05, 0.07)
    assert np.array_equal(a, b)


def test_grouped_query_equals_repeated_kv_heads(orc):
    """GQA with G = 4 equals multi-head attention with each KV head stored
    four times (query head h reads KV head h // G)."""
    rng = np.random.default_rng(14)
    lens = [23, 50]
    Hkv, G = 2, 4
    kp, vp, bt, Ks, Vs = _write_sequences(orc, rng, lens, Hkv, False, 16)
    q = rng.standard_normal((2, Hkv * G, D)).astype(np.float16)
    gqa = orc.paged_attention_decode(q, kp, vp, bt, lens, Hkv, False, 0.1)
    NB = 16
    kp2 = np.zeros(NB * Hkv * G * BS * D * 2, dtype=np.uint8)
    vp2 = kp2.copy()
    for b, L in enumerate(lens):
        k_rep = np.repeat(Ks[b], G, axis=1)
        v_rep = np.repeat(Vs[b], G, axis=1)
        orc.reshape_and_cache(k_rep, v_rep, kp2, vp2, orc.slots_for(bt, [b] * L, range(L)),
                              Hkv * G, False)
    mha = orc.paged_attention_decode(q, kp2, vp2, bt, lens, Hkv * G, False, 0.1)
    assert np.array_equal(gqa, mha)


def test_masked_slots_and_stale_table_entries_are_ignored(orc):
    rng = np.random.default_rng(15)
    lens = [21]
    Hkv, NB, e = 1, 8, 2
    kp, vp, bt, _, _ = _write_sequences(orc, rng, lens, Hkv, False, NB)
    q = rng.standard_normal((1, 2, D)).astype(np.float16)
    out1 = orc.paged_attention_decode(q, kp, vp, bt, lens, Hkv, False, 0.1)
    # scribble over slots 21..31 of the tail block and give the table a stale extra entry
    tile = Hkv * BS * D * e
    tail = bt[0, 1]
    for t in range(5, 16):
        for d in range(D):
            a = (tail * Hkv * BS * D + orc.k_offset(t, d, e)) * e
            kp[a:a + 2] = np.array([7.0], dtype=np.float16).view(np.uint8)
            a = (tail * Hkv * BS * D + orc.v_offset(t, d, e)) * e
            vp[a:a + 2] = np.array([-9.0], dtype=np.float16).view(np.uint8)
    bt2 = np.concatenate([bt, np.array([[int(bt[0, 0])]], dtype=np.int32)], axis=1)
    out2 = orc.paged_attention_decode(q, kp, vp, bt2, lens, Hkv, False, 0.1)
    assert tile > 0
    assert np.array_equal(out1, out2)
