"""Pins of the oracle's block-pool model and sizing formula against the
numbers the pages print."""
import math

import pytest

from conftest import golden


def test_bytes_per_token_llama70b(orc):
    g = golden("kv_sizing.txt")
    args = (int(g["n_layers"]), int(g["n_kv_heads"]), int(g["d_head"]))
    fp16 = orc.bytes_per_token(*args, int(g["fp16_bytes"]))
    assert fp16 == int(g["bytes_per_token_fp16"])
    assert fp16 / 1e6 == pytest.approx(float(g["mb_per_token_printed"]), abs=0.01)
    fp8 = orc.bytes_per_token(*args, 1)
    assert 1 - fp8 / fp16 == float(g["fp8_saving_fraction"])


@pytest.mark.parametrize("which", ["8k", "32k", "128k"])
def test_session_sizes_as_printed(orc, which):
    """The page multiplies the rounded 0.32 MB/token by the context length."""
    g = golden("kv_sizing.txt")
    tokens = int(g[f"session_{which}_tokens"])
    printed = float(g[f"session_{which}_gb_printed"])
    # the page truncates to two decimals (10.4858 is printed as 10.48)
    assert tokens * float(g["mb_per_token_printed"]) / 1000 == pytest.approx(printed, abs=0.01)
    exact = tokens * orc.bytes_per_token(80, 8, 128, 2)
    # the exact figure is a power-of-two multiple of 2.5 GiB worth of tokens
    assert exact == tokens // 8192 * 2_684_354_560
    assert abs(exact / 1e9 - printed) / printed < 0.03   # the rounding the page made


def test_4096_token_sequence_about_1_3_gb(orc):
    g = golden("kv_sizing.txt")
    b = int(g["seq_4096_tokens"]) * orc.bytes_per_token(80, 8, 128, 2)
    assert b / 1e9 == pytest.approx(float(g["seq_4096_gb_printed"]), abs=0.05)


def test_block_table_figure(orc):
    """Physical blocks handed out in the figure's order reproduce its table."""
    g = golden("block_table_figure.txt")
    want = [int(x) for x in g["table_req_a"].split()]
    free = want + [b for b in range(12) if b not in want]
    pool = orc.BlockPoolModel(free)
    a = pool.create()
    slots, pairs = pool.append(a, 48)
    assert pool.table(a) == want and pairs == []
    for tok in (0, 20, 40, 47):
        assert slots[tok] == int(g[f"token_{tok}_slot"])


def test_best_of_8_slots(orc):
    g = golden("sharing.txt")
    P, n, gen = int(g["prompt_tokens"]), int(g["branches"]), int(g["generated_per_branch"])
    bs = 16
    shared = orc.BlockPoolModel(range(4096))
    root = shared.create()
    shared.append(root, P)
    seqs = [root] + [shared.fork(root) for _ in range(n - 1)]
    for s in seqs:
        shared.append(s, gen)
    distinct_tokens = P + n * gen
    assert distinct_tokens == int(g["slots_shared"])
    assert n * (P + gen) == int(g["slots_unshared"])
    used_blocks = shared.num_blocks - shared.num_free()
    assert used_blocks == math.ceil(P / bs) + n * math.ceil(gen / bs)   # 125 + 8*7 = 181
    private = orc.BlockPoolModel(range(4096))
    for _ in range(n):
        s = private.create()
        private.append(s, P + gen)
    assert private.num_blocks - private.num_free() == n * math.ceil((P + gen) / bs)   # 1056
    # the slot capacity held is within one block per sequence of the tokens stored
    assert used_blocks * bs - distinct_tokens <= n * (bs - 1)


def test_four_way_branching_saving_tends_to_75_percent(orc):
    g = golden("sharing.txt")
    ways, limit = int(g["branching_ways"]), float(g["branching_saving_limit"])
    savings = []
    for ctx_blocks in (10, 100, 1000):
        pool = orc.BlockPoolModel(range(8192))
        root = pool.create()
        pool.append(root, ctx_blocks * 16)
        kids = [root] + [pool.fork(root) for _ in range(ways - 1)]
        for k in kids:
            pool.append(k, 16)
        shared = pool.num_blocks - pool.num_free()
        unshared = ways * (ctx_blocks + 1)
        savings.append(1 - shared / unshared)
    assert all(s < limit for s in savings)
    assert savings == sorted(savings) and limit - savings[-1] < 0.001


def test_idle_slots_at_most_one_partial_block(orc):
    g = golden("sharing.txt")
    pool = orc.BlockPoolModel(range(2048))
    import random
    rnd = random.Random(3)
    seqs = [pool.create() for _ in range(40)]
    for s in seqs:
        pool.append(s, rnd.randint(1, 700))
    for s in seqs:
        idle = len(pool.table(s)) * 16 - pool.length(s)
        assert 0 <= idle <= int(g["max_idle_slots_per_seq"])


def test_copy_on_write_of_shared_partial_block(orc):
    pool = orc.BlockPoolModel(range(16))
    a = pool.create()
    pool.append(a, 20)                 # blocks 0, 1 (block 1 partially filled)
    b = pool.fork(a)
    assert pool.ref[0] == 2 and pool.ref[1] == 2
    slots, pairs = pool.append(b, 1)   # b writes into the shared tail: copy it first
    assert pairs == [(1, 2)]
    assert pool.table(b) == [0, 2] and pool.table(a) == [0, 1]
    assert slots == [2 * 16 + 4]
    assert pool.ref[1] == 1 and pool.ref[2] == 1
    slots, pairs = pool.append(a, 1)   # a's tail is private again: no copy
    assert pairs == [] and slots == [1 * 16 + 4]


def test_cancel_returns_every_block(orc):
    pool = orc.BlockPoolModel(range(64))
    a = pool.create()
    pool.append(a, 100)
    kids = [pool.fork(a) for _ in range(3)]
    for k in kids:
        pool.append(k, 30)
    for s in [a] + kids:
        pool.free_seq(s)
    assert pool.num_free() == 64 and all(r == 0 for r in pool.ref)


def test_exhaustion_changes_nothing(orc):
    pool = orc.BlockPoolModel(range(4))
    a = pool.create()
    pool.append(a, 40)                 # 3 blocks
    before = (list(pool.free), list(pool.ref), pool.table(a), pool.length(a))
    with pytest.raises(orc.NoFreeBlocks):
        pool.append(a, 40)             # needs 3 more, 1 free
    assert before == (list(pool.free), list(pool.ref), pool.table(a), pool.length(a))
