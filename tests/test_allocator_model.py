"""Pins of the Python block-pool model (CPU only): page numbers and invariants."""
import json
import os

import numpy as np
import pytest

from oracle.allocator_model import (NO_BLOCKS, INVALID_ARG, STATE, OUT_OF_RANGE, AllocError,
                                    BlockPoolModel)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_block_counts_printed_on_pages():
    with open(os.path.join(GOLDEN, "block_counts.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        m = BlockPoolModel(c["blocks"] + 3, g["block_size"])
        s = m.seq_create()
        m.reserve(s, c["tokens"])
        assert len(m.table(s)) == c["blocks"], c["cite"]
        m.check_invariants()


def test_on_demand_growth_one_block_per_16_tokens():
    # cf-1.com/news/5824798 §3.2: a new block only when the current one is full
    m = BlockPoolModel(8, 16, free_order=[5, 2, 7, 0, 1, 3, 4, 6])
    s = m.seq_create()
    slots = []
    for _ in range(33):
        slots += m.reserve(s, 1)
    assert m.table(s) == [5, 2, 7]
    assert slots[:16] == [5 * 16 + i for i in range(16)]
    assert slots[16:32] == [2 * 16 + i for i in range(16)]
    assert slots[32] == 7 * 16
    assert m.free_list() == [0, 1, 3, 4, 6]


def test_shared_prefix_is_stored_once():
    # cf-1.com/news/5824798 §2.3 and §3.3: a 2048-token system prompt shared by 16
    # requests is kept once; every table points at the same physical blocks
    m = BlockPoolModel(128 + 16 * 10, 16)
    owner = m.seq_create()
    m.reserve(owner, 2048)
    kids = [m.fork(owner, 2048) for _ in range(15)]
    prefix = m.table(owner)
    assert all(m.table(k) == prefix for k in kids)
    assert all(m.refcount(b) == 16 for b in prefix)
    for k in [owner] + kids:
        m.reserve(k, 100)
    used = m.N - len(m.free_list())
    assert used == 128 + 16 * 7            # prefix once + ceil(100/16) own blocks each
    assert m.shared_blocks() == 128
    m.check_invariants()
    for k in kids:
        m.free_seq(k)
    assert all(m.refcount(b) == 1 for b in prefix)
    m.free_seq(owner)
    assert len(m.free_list()) == m.N
    m.check_invariants()


def test_errors_and_atomic_reserve():
    m = BlockPoolModel(4, 16)
    s = m.seq_create()
    m.reserve(s, 40)                                  # 3 blocks
    before = (m.table(s), m.length(s), m.free_list())
    with pytest.raises(AllocError) as e:
        m.reserve(s, 40)                              # needs 3 more, 1 free
    assert e.value.code == NO_BLOCKS
    assert (m.table(s), m.length(s), m.free_list()) == before
    with pytest.raises(AllocError) as e:
        m.fork(s, 48)
    assert e.value.code == INVALID_ARG
    with pytest.raises(AllocError) as e:
        m.tables([s], 2)
    assert e.value.code == OUT_OF_RANGE
    m.free_seq(s)
    with pytest.raises(AllocError) as e:
        m.free_seq(s)
    assert e.value.code == STATE
    with pytest.raises(AllocError) as e:
        BlockPoolModel(4, 16, free_order=[0, 1, 1, 2])
    assert e.value.code == INVALID_ARG


def test_random_traces_keep_invariants():
    rng = np.random.default_rng(0)
    for trial in range(20):
        n = int(rng.integers(8, 65))
        m = BlockPoolModel(n, 16, free_order=rng.permutation(n))
        live = []
        for _ in range(500):
            op = rng.integers(0, 4)
            try:
                if op == 0 or not live:
                    live.append(m.seq_create())
                elif op == 1:
                    m.reserve(live[rng.integers(len(live))], int(rng.integers(0, 40)))
                elif op == 2:
                    p = live[rng.integers(len(live))]
                    live.append(m.fork(p, int(rng.integers(0, m.length(p) + 1))))
                else:
                    m.free_seq(live.pop(rng.integers(len(live))))
            except AllocError as e:
                assert e.code == NO_BLOCKS
            m.check_invariants()


def test_copy_on_write_of_a_shared_partial_block():
    # cf-1.com/news/5824798 §3.3: branches share the prefix blocks; the first to
    # write into a shared block gets a copy of it and writes there
    m = BlockPoolModel(10, 16, free_order=range(10))
    parent = m.seq_create()
    m.reserve(parent, 37)                             # blocks 0, 1, 2 (block 2 holds 5 tokens)
    beams = [m.fork(parent, 37) for _ in range(2)]
    assert all(m.table(b) == [0, 1, 2] for b in beams) and m.refcount(2) == 3
    slot = m.reserve(beams[0], 1)                     # writes position 37 -> copy of block 2
    assert m.table(beams[0]) == [0, 1, 3] and slot == [3 * 16 + 5]
    assert m.take_copies() == [(2, 3)] and m.refcount(2) == 2
    slot = m.reserve(parent, 12)                      # positions 37..48: copy, then one new block
    assert m.table(parent) == [0, 1, 4, 5] and m.take_copies() == [(2, 4)]
    assert slot[:11] == [4 * 16 + 5 + i for i in range(11)] and slot[11] == 5 * 16
    assert m.refcount(2) == 1                         # only beams[1] still holds block 2
    m.reserve(beams[1], 1)                            # sole holder now: writes in place
    assert m.table(beams[1]) == [0, 1, 2] and m.take_copies() == []
    # full blocks stay shared, aligned forks never copy
    assert m.refcount(0) == 3 and m.refcount(1) == 3
    c = m.fork(parent, 32)
    m.reserve(c, 3)
    assert m.table(c)[:2] == [0, 1] and m.take_copies() == []
    m.check_invariants()


def test_copy_on_write_counts_toward_atomic_reserve():
    m = BlockPoolModel(3, 16)
    p = m.seq_create()
    m.reserve(p, 20)                                  # 2 blocks, 1 free
    c = m.fork(p, 20)
    m.reserve(c, 1)                                   # copy takes the last free block
    assert m.free_list() == [] and m.take_copies() == [(1, 2)]
    with pytest.raises(AllocError) as e:
        m.reserve(p, 13)                              # sole holder of block 1 now; needs 1 new block
    assert e.value.code == NO_BLOCKS


def test_splitmix64_published_outputs():
    # Vigna's splitmix64.c seeded with 0: the state advances by the golden gamma
    # before each output; its first outputs are these
    from oracle.allocator_model import splitmix64
    gamma = 0x9E3779B97F4A7C15
    outs = [splitmix64((i * gamma) & ((1 << 64) - 1)) for i in range(4)]
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]


def test_prefix_cache_reuses_and_evicts_lru():
    # cf-1.com/news/5824798 §3.3: a request whose prompt prefix matches reuses the
    # cached blocks; m.lqnn.cn/news/219451 §3: a different identity must miss
    m = BlockPoolModel(6, 16, free_order=range(6))
    prompt = list(range(100, 140))                      # 40 tokens: 2 full blocks + 8
    a = m.seq_create()
    m.reserve(a, 40)
    assert m.prefix_register(a, prompt, ns=7) == 2
    b, hit = m.seq_create_cached(prompt, ns=7)
    assert hit == 32 and m.table(b) == [0, 1] and m.refcount(0) == 2
    c, hit = m.seq_create_cached(prompt, ns=8)          # other namespace: no reuse
    assert hit == 0
    d, hit = m.seq_create_cached(prompt[:16] + [0] * 24, ns=7)
    assert hit == 16 and m.table(d) == [0]              # match stops at the first differing block
    for s in (a, b, c, d):
        m.free_seq(s)
    assert m.free_list() == [3, 4, 5, 2] and m.lru == [1, 0]   # cached blocks wait, LRU order
    e, hit = m.seq_create_cached(prompt, ns=7)          # evictable blocks are taken back
    assert hit == 32 and m.lru == [] and m.refcount(0) == 1
    m.free_seq(e)
    f = m.seq_create()
    m.reserve(f, 16 * 5)                                # 4 free blocks, then evict the oldest cached
    assert m.table(f) == [3, 4, 5, 2, 1] and m.lru == [0]
    g, hit = m.seq_create_cached(prompt, ns=7)          # block 1's content is gone: the chain stops at 0
    assert hit == 16
    m.check_invariants()


def test_prefix_cache_never_shares_on_a_hash_match_alone():
    m = BlockPoolModel(4, 16)
    a = m.seq_create()
    m.reserve(a, 16)
    m.prefix_register(a, list(range(16)))
    key, _ = m.key_of[m.table(a)[0]]
    m.key_of[m.table(a)[0]] = (key, [999] * 16)         # plant stored tokens that differ
    _, hit = m.seq_create_cached(list(range(16)))
    assert hit == 0


def test_swap_out_and_in():
    # cf-1.com/news/5824798 §2.2: inactive blocks may move to host memory and come
    # back on demand; here a whole sequence at a time
    m = BlockPoolModel(8, 16, free_order=range(8))
    a = m.seq_create()
    m.reserve(a, 40)                                  # blocks 0, 1, 2
    b = m.fork(a, 32)                                 # shares 0, 1
    assert m.swap_out(a) == 3
    assert m.free_list() == [3, 4, 5, 6, 7, 2]        # only its private block came free
    assert m.refcount(0) == 1 and m.length(a) == 40
    for op in (lambda: m.reserve(a, 1), lambda: m.fork(a, 1), lambda: m.table(a), lambda: m.swap_out(a)):
        with pytest.raises(AllocError) as e:
            op()
        assert e.value.code == STATE
    assert m.swap_in(a) == [3, 4, 5]                  # fresh private copies, logical order
    assert m.table(b) == [0, 1] and m.refcount(0) == 1
    m.reserve(a, 9)                                   # grows normally afterwards
    assert m.table(a) == [3, 4, 5, 6]
    with pytest.raises(AllocError) as e:
        m.swap_in(a)                                  # not swapped out
    assert e.value.code == STATE
    c = m.seq_create()
    m.reserve(c, 32)                                  # the last two free blocks
    assert m.table(c) == [7, 2] and m.free_list() == []
    m.check_invariants()


def test_swap_in_is_all_or_nothing():
    m = BlockPoolModel(4, 16)
    a = m.seq_create()
    m.reserve(a, 64)
    m.swap_out(a)
    b = m.seq_create()
    m.reserve(b, 16)                                  # one of the four blocks is taken
    before = m.free_list()
    with pytest.raises(AllocError) as e:
        m.swap_in(a)
    assert e.value.code == NO_BLOCKS and m.free_list() == before and a in m.swapped
    m.free_seq(b)
    assert len(m.swap_in(a)) == 4
    m.free_seq(a)                                     # a swapped or resident sequence frees alike
    m.check_invariants()
