"""Pins of the oracle's FP8 write and decode with per-block dynamic scales
("Optimización de KV Cache con PagedAttention y Cuantización FP8 ... (128K)",
§8: the GPU measures the MaxAbs of each cache block as it writes and scales by
it).  Expected codes come from numpy's IEEE fp32 division and torch's
float8_e4m3fn cast, expected attention from torch SDPA in fp64; closed forms
cover growth of a block's scale and the fresh-block reset."""
import math

import numpy as np
import pytest
import torch

BS, D = 16, 128
FLOOR = np.float32(2.0 ** -126)


def _offsets(orc):
    k = np.array([[orc.k_offset(t, d, 1) for d in range(D)] for t in range(BS)], dtype=np.int64)
    v = np.array([[orc.v_offset(t, d, 1) for d in range(D)] for t in range(BS)], dtype=np.int64)
    return k, v


def _rows(pool, off, blk, h, Hkv):
    """[BS][D] codes of one (block, head) tile, read through the layout."""
    base = (blk * Hkv + h) * BS * D
    return pool[base + off]


def _cast(u32):
    """Library E4M3FN codes of fp32 values."""
    return torch.from_numpy(np.ascontiguousarray(u32, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _value(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def _empty(NB, Hkv, fill=0):
    n = NB * Hkv * BS * D
    return (np.full(n, fill, np.uint8), np.full(n, fill, np.uint8),
            np.zeros((NB, Hkv), np.float32), np.zeros((NB, Hkv), np.float32))


def test_one_call_fill_matches_library_cast(orc):
    """Whole blocks written in one call: scale = fp32(MaxAbs / 448) per
    (block, head), codes = library cast of fp32(x / scale)."""
    rng = np.random.default_rng(1)
    NB, Hkv = 5, 3
    kp, vp, ks, vs = _empty(NB, Hkv, 0xA5)
    blocks = [3, 0, 4]
    slots = np.array([b * BS + t for b in blocks for t in range(BS)], np.int64)
    key = (rng.standard_normal((len(slots), Hkv, D)) * rng.uniform(0.1, 8, (1, Hkv, 1))
           ).astype(np.float16)
    val = (rng.standard_normal((len(slots), Hkv, D)) * 0.3).astype(np.float16)
    orc.reshape_and_cache_dynamic(key, val, kp, vp, ks, vs, slots, Hkv)
    koff, voff = _offsets(orc)
    for i, b in enumerate(blocks):
        rows = slice(i * BS, (i + 1) * BS)
        for h in range(Hkv):
            for src, pool, sc, off in ((key, kp, ks, koff), (val, vp, vs, voff)):
                x = src[rows, h, :].astype(np.float32)
                s = max(np.float32(np.abs(x).max()) / np.float32(448.0), FLOOR)
                assert sc[b, h] == s
                assert np.array_equal(_rows(pool, off, b, h, Hkv), _cast(x / s))
    # untouched blocks keep their bytes and scales
    for b in (1, 2):
        assert (ks[b] == 0).all() and (vs[b] == 0).all()
        base = b * Hkv * BS * D
        assert (kp[base:base + Hkv * BS * D] == 0xA5).all()


def test_largest_element_maps_to_448_and_error_is_within_half_a_step(orc):
    rng = np.random.default_rng(2)
    NB, Hkv = 2, 2
    kp, vp, ks, vs = _empty(NB, Hkv)
    x = (rng.standard_normal((BS, Hkv, D)) * 3).astype(np.float16)
    orc.reshape_and_cache_dynamic(x, x, kp, vp, ks, vs, np.arange(BS, dtype=np.int64) + BS, Hkv)
    koff, _ = _offsets(orc)
    for h in range(Hkv):
        codes = _rows(kp, koff, 1, h, Hkv)
        xs = x[:, h, :].astype(np.float64)
        i = np.unravel_index(np.argmax(np.abs(xs)), xs.shape)
        assert codes[i] & 0x7F == 0x7E                        # +-448
        got = _value(codes) * float(ks[1, h])
        # E4M3 keeps 3 mantissa bits (relative half step 2^-4) and a subnormal
        # grid of 2^-9, both in units of the scale
        assert (np.abs(got - xs) <= np.abs(xs) * 2.0 ** -4 + float(ks[1, h]) * 2.0 ** -10).all()


def test_growth_by_a_power_of_two_requantizes_old_rows_exactly(orc):
    """Token 0 holds codes whose value is exact at scale 2^-4; token 1 doubles
    the block's MaxAbs, so the scale becomes 2^-3 and every old normal code
    drops exactly one binade (code - 8)."""
    NB, Hkv = 3, 1
    kp, vp, ks, vs = _empty(NB, Hkv)
    rng = np.random.default_rng(3)
    codes0 = rng.integers(0x10, 0x7E, D).astype(np.uint8)        # exponent field >= 2
    codes0[5] = 0x7E                                             # the MaxAbs: 448 * 2^-4 = 28
    codes0[9] |= 0x80                                            # one negative
    x0 = (_value(codes0) * 2.0 ** -4).astype(np.float16)
    assert np.array_equal(x0.astype(np.float64), _value(codes0) * 2.0 ** -4)
    row0 = x0.reshape(1, 1, D)
    orc.reshape_and_cache_dynamic(row0, row0, kp, vp, ks, vs, np.array([2 * BS], np.int64), Hkv)
    assert ks[2, 0] == np.float32(2.0 ** -4)
    koff, voff = _offsets(orc)
    assert np.array_equal(_rows(kp, koff, 2, 0, Hkv)[0], codes0)
    x1 = (rng.standard_normal(D) * 10).astype(np.float16)
    x1[0] = 56.0                                                 # 448 * 2^-3
    x1 = np.clip(x1, -56, 56).astype(np.float16).reshape(1, 1, D)
    orc.reshape_and_cache_dynamic(x1, x1, kp, vp, ks, vs, np.array([2 * BS + 1], np.int64), Hkv)
    assert ks[2, 0] == np.float32(2.0 ** -3) and vs[2, 0] == np.float32(2.0 ** -3)
    for pool, off in ((kp, koff), (vp, voff)):
        tile = _rows(pool, off, 2, 0, Hkv)
        assert np.array_equal(tile[0], codes0 - 8)
        assert np.array_equal(tile[1], _cast(x1[0, 0].astype(np.float32) / np.float32(0.125)))


def test_growth_keeps_old_rows_within_two_roundings(orc):
    rng = np.random.default_rng(4)
    NB, Hkv = 2, 2
    kp, vp, ks, vs = _empty(NB, Hkv)
    xs = (rng.standard_normal((6, Hkv, D)) * np.array([1, 1.3, 2.2, 0.5, 4.1, 3.0])[:, None, None]
          ).astype(np.float16)
    for t in range(6):                      # one token per call, scale grows at t = 1, 2, 4
        orc.reshape_and_cache_dynamic(xs[t:t + 1], xs[t:t + 1], kp, vp, ks, vs,
                                      np.array([BS + t], np.int64), Hkv)
    koff, _ = _offsets(orc)
    for h in range(Hkv):
        s = float(ks[1, h])
        assert ks[1, h] == np.float32(np.abs(xs[:, h].astype(np.float32)).max()) / np.float32(448)
        got = _value(_rows(kp, koff, 1, h, Hkv)[:6]) * s
        x = xs[:, h, :].astype(np.float64)
        # each growth re-rounds once more: at most 3 roundings of half a step
        bound = 3 * (np.abs(x) * 2.0 ** -4 * 1.07 + s * 2.0 ** -10)
        assert (np.abs(got - x) <= bound).all()
        # the newest row was rounded once, at the final scale
        assert np.array_equal(_rows(kp, koff, 1, h, Hkv)[5],
                              _cast(xs[5, h].astype(np.float32) / ks[1, h]))


def test_no_growth_means_token_by_token_equals_one_call(orc):
    rng = np.random.default_rng(5)
    NB, Hkv = 4, 2
    x = (rng.standard_normal((BS, Hkv, D))).astype(np.float16)
    x[0] *= 8                               # the first token holds each head's MaxAbs
    slots = np.arange(BS, dtype=np.int64) + 2 * BS
    a = _empty(NB, Hkv)
    orc.reshape_and_cache_dynamic(x, x, *a, slots, Hkv)
    b = _empty(NB, Hkv)
    for t in range(BS):
        orc.reshape_and_cache_dynamic(x[t:t + 1], x[t:t + 1], *b, slots[t:t + 1], Hkv)
    for u, w in zip(a, b):
        assert np.array_equal(u, w)


def test_offset_zero_starts_a_fresh_block(orc):
    """A reused block: writing its first slot disregards the stale scale and
    leaves the stale bytes of other slots alone."""
    NB, Hkv = 2, 1
    kp, vp, ks, vs = _empty(NB, Hkv, 0x33)
    ks[:] = 1000.0
    vs[:] = 1000.0
    x = np.full((1, 1, D), 0.5, np.float16)
    x[0, 0, 7] = -2.0
    orc.reshape_and_cache_dynamic(x, x, kp, vp, ks, vs, np.array([BS], np.int64), Hkv)
    assert ks[1, 0] == np.float32(2.0) / np.float32(448.0) and ks[0, 0] == 1000.0
    koff, _ = _offsets(orc)
    tile = _rows(kp, koff, 1, 0, Hkv)
    assert (tile[1:] == 0x33).all()
    assert tile[0, 7] == 0xFE and tile[0, 0] == _cast(np.float32(0.5) / ks[1, 0])
    # a later token in the same block grows the scale from the new value
    y = np.full((1, 1, D), 4.0, np.float16)
    orc.reshape_and_cache_dynamic(y, y, kp, vp, ks, vs, np.array([BS + 1], np.int64), Hkv)
    assert ks[1, 0] == np.float32(4.0) / np.float32(448.0)
    tile = _rows(kp, koff, 1, 0, Hkv)
    assert tile[0, 7] == 0xF6                   # -448 * 1/2 = -224
    assert tile[1, 0] == 0x7E


def test_zero_rows_get_the_floor_scale_and_non_finite_values_are_not_measured(orc):
    NB, Hkv = 2, 1
    kp, vp, ks, vs = _empty(NB, Hkv)
    z = np.zeros((1, 1, D), np.float16)
    orc.reshape_and_cache_dynamic(z, z, kp, vp, ks, vs, np.array([0], np.int64), Hkv)
    assert ks[0, 0] == FLOOR and vs[0, 0] == FLOOR
    koff, _ = _offsets(orc)
    assert (_rows(kp, koff, 0, 0, Hkv)[0] == 0).all()
    x = np.full((1, 1, D), 1.0, np.float16)
    x[0, 0, 0], x[0, 0, 1], x[0, 0, 2] = np.inf, -np.inf, np.nan
    orc.reshape_and_cache_dynamic(x, x, kp, vp, ks, vs, np.array([BS], np.int64), Hkv)
    assert ks[1, 0] == np.float32(1.0) / np.float32(448.0)
    row = _rows(kp, koff, 1, 0, Hkv)[0]
    assert row[0] == 0x7E and row[1] == 0xFE and row[2] & 0x7F == 0x7F and row[3] == 0x7E


def _dynamic_sequences(orc, rng, lens, Hkv, NB, calls=3):
    """Sequences written in a few calls each (growing scales included)."""
    perm = rng.permutation(NB).astype(np.int32)
    nblk = [-(-L // BS) for L in lens]
    bt = np.zeros((len(lens), max(nblk)), np.int32)
    pos = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    kp, vp, ks, vs = _empty(NB, Hkv, 0x21)
    for b, L in enumerate(lens):
        k = (rng.standard_normal((L, Hkv, D)) * rng.uniform(0.2, 3, (L, 1, 1))).astype(np.float16)
        v = (rng.standard_normal((L, Hkv, D)) * rng.uniform(0.2, 3, (L, 1, 1))).astype(np.float16)
        cuts = sorted(set([0, L] + list(rng.integers(0, L + 1, calls - 1))))
        for c0, c1 in zip(cuts[:-1], cuts[1:]):
            sl = orc.slots_for(bt, [b] * (c1 - c0), range(c0, c1))
            orc.reshape_and_cache_dynamic(k[c0:c1], v[c0:c1], kp, vp, ks, vs, sl, Hkv)
    return kp, vp, ks, vs, bt


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (6, 3)])
def test_decode_with_block_scales_matches_library_sdpa(orc, Hq, Hkv):
    """Rows rebuilt from the pool bytes through the layout and the library's
    E4M3 view, times their own (block, head) scale, into torch SDPA."""
    rng = np.random.default_rng(20 + Hq)
    lens = [1, 16, 17, 40, 75]
    NB = 32
    kp, vp, ks, vs, bt = _dynamic_sequences(orc, rng, lens, Hkv, NB)
    assert len(np.unique(ks)) > NB // 2         # the scales really differ
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float16)
    sm = np.float32(1 / math.sqrt(D))
    got = orc.paged_attention_decode_dynamic(q, kp, vp, ks, vs, bt, lens, Hkv, sm)
    koff, voff = _offsets(orc)
    G = Hq // Hkv
    for b, L in enumerate(lens):
        K = np.zeros((Hkv, L, D))
        V = np.zeros((Hkv, L, D))
        for t in range(L):
            blk = int(bt[b, t // BS])
            for h in range(Hkv):
                K[h, t] = _value(_rows(kp, koff, blk, h, Hkv)[t % BS]) * float(ks[blk, h])
                V[h, t] = _value(_rows(vp, voff, blk, h, Hkv)[t % BS]) * float(vs[blk, h])
        k = torch.from_numpy(K).repeat_interleave(G, dim=0)
        v = torch.from_numpy(V).repeat_interleave(G, dim=0)
        qq = torch.from_numpy(q[b].astype(np.float64)).unsqueeze(1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0), scale=float(sm))[0, :, 0, :].numpy()
        assert np.max(np.abs(got[b] - ref)) < 1e-12


def test_uniform_block_scales_equal_the_per_tensor_decode(orc):
    rng = np.random.default_rng(30)
    Hkv, NB, lens = 2, 16, [5, 33, 64]
    kp, vp, ks, vs, bt = _dynamic_sequences(orc, rng, lens, Hkv, NB)
    s = np.float32(0.0173)
    q = rng.standard_normal((len(lens), 8, D)).astype(np.float16)
    sm = np.float32(1 / math.sqrt(D))
    got = orc.paged_attention_decode_dynamic(q, kp, vp, np.full_like(ks, s), np.full_like(vs, s),
                                             bt, lens, Hkv, sm)
    ref = orc.paged_attention_decode(q, kp, vp, bt, lens, Hkv, True, sm, s, s)
    assert np.array_equal(got, ref)


# ------------------------------------------- chunked prefill over block scales

def _rebuilt_rows(orc, kp, vp, ks, vs, bt, b, L, Hkv):
    """Sequence b's K and V [Hkv][L][D] from the pool bytes, through the layout
    and the library's E4M3 view, each times its own (block, head) scale."""
    koff, voff = _offsets(orc)
    K = np.zeros((Hkv, L, D))
    V = np.zeros((Hkv, L, D))
    for t in range(L):
        blk = int(bt[b, t // BS])
        for h in range(Hkv):
            K[h, t] = _value(_rows(kp, koff, blk, h, Hkv)[t % BS]) * float(ks[blk, h])
            V[h, t] = _value(_rows(vp, voff, blk, h, Hkv)[t % BS]) * float(vs[blk, h])
    return K, V


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (6, 3)])
def test_prefill_with_block_scales_matches_library_sdpa(orc, Hq, Hkv):
    """Each sequence's last chunk attends causally over rows rebuilt with their
    own block's scales, in torch SDPA with an explicit causal mask."""
    rng = np.random.default_rng(40 + Hq)
    lens = [1, 16, 17, 40, 75]
    n = [1, 5, 17, 0, 40]                       # whole sequences, ragged, empty
    kp, vp, ks, vs, bt = _dynamic_sequences(orc, rng, lens, Hkv, 32)
    assert len(np.unique(vs)) > 8
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), Hq, D)).astype(np.float16)
    sm = np.float32(1 / math.sqrt(D))
    got = orc.paged_prefill_attention_dynamic(q, kp, vp, ks, vs, bt, lens, qs, Hkv, sm)
    G = Hq // Hkv
    for b, L in enumerate(lens):
        if n[b] == 0:
            continue
        K, V = _rebuilt_rows(orc, kp, vp, ks, vs, bt, b, L, Hkv)
        k = torch.from_numpy(K).repeat_interleave(G, dim=0)
        v = torch.from_numpy(V).repeat_interleave(G, dim=0)
        qq = torch.from_numpy(q[qs[b]:qs[b + 1]].astype(np.float64)).permute(1, 0, 2)
        pos = L - n[b] + np.arange(n[b])
        mask = torch.from_numpy(np.arange(L)[None, :] <= pos[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0), attn_mask=mask,
            scale=float(sm))[0].permute(1, 0, 2).numpy()
        assert np.max(np.abs(got[qs[b]:qs[b + 1]] - ref)) < 1e-12


def test_prefill_with_block_scales_rows_are_the_dynamic_decode_of_their_prefix(orc):
    rng = np.random.default_rng(41)
    lens, Hkv, Hq = [37, 64], 2, 8
    kp, vp, ks, vs, bt = _dynamic_sequences(orc, rng, lens, Hkv, 16)
    n = [20, 64]
    qs = np.array([0, 20, 84], np.int32)
    q = rng.standard_normal((84, Hq, D)).astype(np.float16)
    sm = np.float32(0.09)
    got = orc.paged_prefill_attention_dynamic(q, kp, vp, ks, vs, bt, lens, qs, Hkv, sm)
    for b, L in enumerate(lens):
        for i in range(n[b]):
            r, p = qs[b] + i, L - n[b] + i
            dec = orc.paged_attention_decode_dynamic(q[r:r + 1], kp, vp, ks, vs, bt[b:b + 1],
                                                     [p + 1], Hkv, sm)
            assert np.array_equal(got[r], dec[0])


def test_prefill_with_uniform_block_scales_equals_the_per_tensor_prefill(orc):
    rng = np.random.default_rng(42)
    Hkv, lens = 2, [5, 33, 64]
    kp, vp, ks, vs, bt = _dynamic_sequences(orc, rng, lens, Hkv, 16)
    qs = np.array([0, 5, 15, 79], np.int32)
    q = rng.standard_normal((79, 8, D)).astype(np.float16)
    sm = np.float32(1 / math.sqrt(D))
    sk, sv = np.float32(0.0173), np.float32(0.031)
    got = orc.paged_prefill_attention_dynamic(q, kp, vp, np.full_like(ks, sk),
                                              np.full_like(vs, sv), bt, lens, qs, Hkv, sm)
    ref = orc.paged_prefill_attention(q, kp, vp, bt, lens, qs, Hkv, True, sm, sk, sv)
    assert np.array_equal(got, ref)
