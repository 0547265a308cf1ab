"""Pins of the oracle's chunked-prefill attention ("Optimización de KV Cache
... (128K)", §5: a long prompt is processed in chunks of tokens; each chunk
attends causally over everything already in the paged cache).

Expected values come from torch SDPA (fp64, CPU) with an explicit causal mask
over the logically ordered rows, from the (separately pinned) decode oracle
at every prefix length, and from causality itself."""
import math

import numpy as np
import pytest
import torch

from test_oracle_attention import _dequant, _write_sequences

BS, D = 16, 128


def _chunks(rng, lens, max_chunk):
    """Each sequence's last n_b tokens form its chunk (0 <= n_b <= L_b)."""
    n = [int(rng.integers(0, min(L, max_chunk) + 1)) for L in lens]
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    return n, qs


def _sdpa_chunks(q, Ks, Vs, lens, n, qs, Hkv, sm, fp8, ks, vs):
    R, Hq, _ = q.shape
    G = Hq // Hkv
    out = np.zeros((R, Hq, D))
    for b, L in enumerate(lens):
        if n[b] == 0:
            continue
        k = _dequant(Ks[b], ks, fp8).permute(1, 0, 2).repeat_interleave(G, dim=0)
        v = _dequant(Vs[b], vs, fp8).permute(1, 0, 2).repeat_interleave(G, dim=0)
        qq = torch.from_numpy(q[qs[b]:qs[b + 1]].astype(np.float64)).permute(1, 0, 2)
        pos = L - n[b] + np.arange(n[b])
        mask = torch.from_numpy(np.arange(L)[None, :] <= pos[:, None])
        o = torch.nn.functional.scaled_dot_product_attention(
            qq.unsqueeze(0), k.unsqueeze(0).contiguous(), v.unsqueeze(0).contiguous(),
            attn_mask=mask, scale=float(np.float32(sm)))
        out[qs[b]:qs[b + 1]] = o[0].permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (6, 3), (4, 4)])
def test_prefill_matches_library_sdpa_with_causal_mask(orc, fp8, Hq, Hkv):
    rng = np.random.default_rng(300 + Hq + 10 * Hkv + int(fp8))
    lens = [1, 5, 16, 17, 40, 70]
    ks, vs = (np.float32(0.011), np.float32(0.013)) if fp8 else (1.0, 1.0)
    kp, vp, bt, Ks, Vs = _write_sequences(orc, rng, lens, Hkv, fp8, 64, ks, vs)
    n, qs = _chunks(rng, lens, 40)
    n[3] = 17                                   # the whole sequence is the chunk
    n[5] = 33
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), Hq, D)).astype(np.float16)
    sm = np.float32(1 / math.sqrt(D))
    got = orc.paged_prefill_attention(q, kp, vp, bt, lens, qs, Hkv, fp8, sm, ks, vs)
    ref = _sdpa_chunks(q, Ks, Vs, lens, n, qs, Hkv, sm, fp8, ks, vs)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_every_chunk_row_is_the_decode_of_its_prefix(orc):
    rng = np.random.default_rng(7)
    lens, Hkv, Hq = [37, 64], 2, 8
    kp, vp, bt, _, _ = _write_sequences(orc, rng, lens, Hkv, True, 16, 0.02, 0.03)
    n = [20, 64]
    qs = np.array([0, 20, 84], np.int32)
    q = rng.standard_normal((84, Hq, D)).astype(np.float16)
    sm = np.float32(0.09)
    got = orc.paged_prefill_attention(q, kp, vp, bt, lens, qs, Hkv, True, sm, 0.02, 0.03)
    for b, L in enumerate(lens):
        for i in range(n[b]):
            r = qs[b] + i
            p = L - n[b] + i
            dec = orc.paged_attention_decode(q[r:r + 1], kp, vp, bt[b:b + 1], [p + 1], Hkv, True,
                                             sm, 0.02, 0.03)
            assert np.max(np.abs(got[r] - dec[0])) < 1e-12


def test_future_tokens_do_not_leak(orc):
    """Changing the keys and values after a row's position changes nothing for
    that row; changing its own position's does."""
    rng = np.random.default_rng(8)
    lens, Hkv, Hq = [48], 1, 2
    kp, vp, bt, _, _ = _write_sequences(orc, rng, lens, Hkv, False, 8, fill_garbage=False)
    qs = np.array([0, 48], np.int32)
    q = rng.standard_normal((48, Hq, D)).astype(np.float16)
    base = orc.paged_prefill_attention(q, kp, vp, bt, lens, qs, Hkv, False, 0.1)
    p = 29
    k2, v2 = kp.copy(), vp.copy()
    new = rng.standard_normal((48 - p - 1, Hkv, D)).astype(np.float16)
    orc.reshape_and_cache(new, new, k2, v2, orc.slots_for(bt, [0] * len(new), range(p + 1, 48)),
                          Hkv, False)
    after = orc.paged_prefill_attention(q, k2, v2, bt, lens, qs, Hkv, False, 0.1)
    assert np.array_equal(after[:p + 1], base[:p + 1])
    assert not np.allclose(after[p + 1:], base[p + 1:])
    one = rng.standard_normal((1, Hkv, D)).astype(np.float16)
    orc.reshape_and_cache(one, one, k2, v2, orc.slots_for(bt, [0], [p]), Hkv, False)
    again = orc.paged_prefill_attention(q, k2, v2, bt, lens, qs, Hkv, False, 0.1)
    assert np.array_equal(again[:p], base[:p]) and not np.allclose(again[p], base[p])


def test_single_token_chunks_equal_decode(orc):
    rng = np.random.default_rng(9)
    lens, Hkv, Hq = [3, 16, 50], 2, 4
    kp, vp, bt, _, _ = _write_sequences(orc, rng, lens, Hkv, True, 16, 0.05, 0.05)
    qs = np.arange(4, dtype=np.int32)
    q = rng.standard_normal((3, Hq, D)).astype(np.float16)
    got = orc.paged_prefill_attention(q, kp, vp, bt, lens, qs, Hkv, True, 0.08, 0.05, 0.05)
    dec = orc.paged_attention_decode(q, kp, vp, bt, lens, Hkv, True, 0.08, 0.05, 0.05)
    assert np.max(np.abs(got - dec)) < 1e-12


def test_empty_chunks_and_rows_before_the_sequence(orc):
    rng = np.random.default_rng(10)
    lens, Hkv, Hq = [10, 20], 1, 1
    kp, vp, bt, _, _ = _write_sequences(orc, rng, lens, Hkv, False, 8)
    qs = np.array([0, 0, 24], np.int32)         # no rows for sequence 0; 24 rows > 20 tokens
    q = rng.standard_normal((24, Hq, D)).astype(np.float16)
    got = orc.paged_prefill_attention(q, kp, vp, bt, lens, qs, Hkv, False, 0.1)
    assert (got[:4] == 0).all()                 # positions -4 .. -1 see nothing
    dec = orc.paged_attention_decode(q[4:5], kp, vp, bt[1:2], [1], Hkv, False, 0.1)
    assert np.max(np.abs(got[4] - dec[0])) < 1e-12
