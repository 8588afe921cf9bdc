"""Pins of the oracle's prefix cache (page 3, section 04) against the page's
two-request example, hand-derived consequences of the LRU reading, closed
forms, and the defining property: a sequence's table shows, at every
position, K/V computed from exactly its own token prefix, whether the
position was written for it or found in the cache."""

import itertools
import json
import os
import random

import pytest

from oracle import AllocError, BlockAllocatorModel, E_NOBLOCKS
from tests.alloc_checks import PrefixWorld, check


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _check_world(m: BlockAllocatorModel, w: PrefixWorld):
    live = list(m.seqs)
    check(w, {s: m.table(s) for s in live}, {s: m.length(s) for s in live},
          m.ref_counts(), m.free_list())
    free = set(m.free_list())
    for key, b in m.cache.items():
        assert m.block_key[b] == key
        assert m.ref[b] > 0 or b in free, "a cached block is referenced or waits in the free list"
        assert w.block_holds(b, key), f"cached block {b} does not hold the K/V of its key"
    assert len(m.block_key) == len(m.cache)


def test_page_example(golden_dir):
    g = _load(golden_dir, "prefix_cache_system_prompt.json")
    m = BlockAllocatorModel(g["num_blocks"], g["block_size"], g["free_order"], prefix_caching=True)
    w = PrefixWorld(g["num_blocks"], g["block_size"])
    for op in g["ops"]:
        e = op["expect"]
        slots, cached = m.add_tokens(op["seq"], op["tokens"])
        assert slots == e["slots"] and cached == e["num_cached"]
        assert m.table(op["seq"]) == e["table"]
        assert {k: m.ref_counts()[int(k)] for k in e["ref_cnt"]} == e["ref_cnt"]
        w.on_add_tokens(op["seq"], op["tokens"], slots, cached)
        _check_world(m, w)
    assert m.free_list() == g["final"]["free"]
    assert m.cache_stats() == g["final"]["stats"]


def test_lru_release_order_revival_and_eviction(golden_dir):
    """Continuation of the page's example under the LRU reading, derived by hand."""
    g = _load(golden_dir, "prefix_cache_system_prompt.json")
    m = BlockAllocatorModel(g["num_blocks"], g["block_size"], g["free_order"], prefix_caching=True)
    sysp = g["ops"][0]["tokens"][:16]
    for op in g["ops"]:
        m.add_tokens(op["seq"], op["tokens"])
    m.free_seq(1)            # blocks 0 (count 0) then 3 (count 1)
    m.free_seq(2)            # blocks 1 then 3: both reach 0
    assert m.free_list() == [2, 4, 5, 6, 7, 0, 1, 3]
    assert m.cached_blocks(sysp + [9]) == [3], "a released block stays cached"
    slots, cached = m.add_tokens(3, sysp + [301, 302, 303])
    assert cached == 16 and m.table(3) == [3, 2], "the hit takes block 3 back out of the free list"
    assert m.free_list() == [4, 5, 6, 7, 0, 1]
    m.free_seq(3)
    assert m.free_list() == [4, 5, 6, 7, 0, 1, 2, 3]
    m.add(4, 8 * 16)         # takes the whole pool: block 3 goes last and loses its entry
    assert m.table(4) == [4, 5, 6, 7, 0, 1, 2, 3]
    assert m.cache_stats()["evictions"] == 1 and m.cache == {}
    m.free_seq(4)
    _, cached = m.add_tokens(5, sysp)
    assert cached == 0 and m.table(5) == [3]
    assert m.cache_stats() == {"hits": 2, "queries": 4, "cached_blocks": 1, "evictions": 1}


def test_least_recently_released_is_evicted_first():
    B = 4
    m = BlockAllocatorModel(6, B, prefix_caching=True)
    a, b = [1] * 8, [2] * 8
    m.add_tokens(1, a)       # blocks 0, 1
    m.add_tokens(2, b)       # blocks 2, 3
    m.free_seq(1)            # released first: 1, 0
    m.free_seq(2)            # then 3, 2
    assert m.free_list() == [4, 5, 1, 0, 3, 2]
    m.add(3, 4 * B)          # takes 4, 5, 1, 0: evicts prompt a's blocks only
    assert m.cached_blocks(a) == [] and m.cached_blocks(b) == [2, 3]
    _, cached = m.add_tokens(4, b)
    assert cached == 8 and m.table(4) == [2, 3] and m.free_list() == []


def test_closed_form_shared_system_prompt():
    """R prompts = the same P full blocks + a unique suffix of L_r tokens, pool
    large enough that nothing is evicted: hits = (R-1)P, every prompt after
    the first finds P*B cached positions, and the pool holds P + sum
    ceil(L_r / B) blocks."""
    B, P, R = 16, 5, 9
    rng = random.Random(3)
    sysp = [rng.randrange(1000) for _ in range(P * B)]
    m = BlockAllocatorModel(4096, B, prefix_caching=True)
    suffix_lens = [rng.randrange(0, 70) for _ in range(R)]
    queries = 0
    for r, L in enumerate(suffix_lens):
        toks = sysp + [10_000 + 100 * r + i for i in range(L)]
        _, cached = m.add_tokens(r, toks)
        assert cached == (0 if r == 0 else P * B)
        queries += len(toks) // B
    st = m.cache_stats()
    assert st["hits"] == (R - 1) * P and st["queries"] == queries
    used = sum(1 for c in m.ref_counts() if c > 0)
    assert used == P + sum(-(-L // B) for L in suffix_lens)
    for blk in m.table(0)[:P]:
        assert m.ref_counts()[blk] == R


def test_no_blocks_counts_revived_hits_and_changes_nothing():
    B = 2
    m = BlockAllocatorModel(3, B, prefix_caching=True)
    m.add_tokens(1, [5, 6, 7, 8])            # blocks 0, 1, both entered
    m.free_seq(1)                            # free: 2, 1, 0 -- 0 and 1 still cached
    before = (m.free_list(), m.ref_counts(), dict(m.cache), m.cache_stats())
    # hits 0 and 1 (both revived) plus 2 fresh blocks: 4 taken off a list of 3
    with pytest.raises(AllocError) as ei:
        m.add_tokens(2, [5, 6, 7, 8, 9, 9, 9])
    assert ei.value.code == E_NOBLOCKS and ei.value.needed == 4 and ei.value.free == 3
    assert (m.free_list(), m.ref_counts(), dict(m.cache), m.cache_stats()) == before
    _, cached = m.add_tokens(2, [5, 6, 7, 8, 9])
    assert cached == 4 and m.table(2) == [0, 1, 2]


def test_disabled_cache_is_plain_allocation():
    B = 4
    on = BlockAllocatorModel(8, B, prefix_caching=False)
    ref = BlockAllocatorModel(8, B)
    toks = [1, 2, 3, 4, 5]
    for s in range(2):
        slots, cached = on.add_tokens(s, toks)
        assert cached == 0 and slots == ref.add(s, len(toks))
    assert on.cache == {} and on.cached_blocks(toks) == []


def test_generated_blocks_are_entered():
    """A block filled by appends that carry ids is entered when its last slot
    is handed out; a sequence that appends without an id stops entering."""
    B = 2
    m = BlockAllocatorModel(8, B, prefix_caching=True)
    m.add_tokens(1, [1])
    m.append(1, 2)                           # fills block 0 = [1, 2]
    assert m.cached_blocks([1, 2]) == [m.table(1)[0]]
    m.append(1, 3)
    m.append(1)                              # id unknown: block [3, ?] is not entered
    assert m.cached_blocks([1, 2, 3, 4]) == [m.table(1)[0]]
    m.append(1, 5)
    m.append(1, 6)
    assert len(m.cache) == 1


def _random_ops(m, w, rng, steps, alphabet, max_prompt):
    B = m.block_size
    next_id = 0
    for _ in range(steps):
        live = sorted(m.seqs)
        r = rng.random()
        try:
            if r < 0.3 or not live:
                n = rng.randrange(0, max_prompt)
                # prompts often start like an earlier one
                if live and rng.random() < 0.6:
                    base = w.tokens[rng.choice(live)]
                    toks = base[:rng.randrange(0, len(base) + 1)]
                    toks = toks + [rng.choice(alphabet) for _ in range(max(0, n - len(toks)))]
                else:
                    toks = [rng.choice(alphabet) for _ in range(n)]
                slots, cached = m.add_tokens(next_id, toks)
                assert cached % B == 0 and cached <= len(toks)
                w.on_add_tokens(next_id, toks, slots, cached)
                next_id += 1
            elif r < 0.4:
                parent = rng.choice(live)
                m.fork(parent, next_id)
                w.on_fork(parent, next_id)
                next_id += 1
            elif r < 0.75:
                seqs = rng.sample(live, rng.randrange(1, len(live) + 1))
                toks = [rng.choice(alphabet) for _ in seqs]
                slots, pairs = m.step(seqs, toks)
                for src, dst in pairs:
                    w.on_copy(src, dst)
                for s, t, sl in zip(seqs, toks, slots):
                    w.on_append_token(s, t, sl)
            else:
                s = rng.choice(live)
                m.free_seq(s)
                w.on_free(s)
        except AllocError as e:
            assert e.code == E_NOBLOCKS
        _check_world(m, w)



@pytest.mark.parametrize("seed", range(12))
def test_random_streams_keep_every_prefix_right(seed):
    """Tiny alphabets and pools: hits, revivals, evictions and copy-on-write
    all happen often; after every call each sequence must read its own
    prefixes and every cached block must hold the K/V of its key."""
    rng = random.Random(seed)
    B = rng.choice([1, 2, 3, 4])
    N = rng.randrange(4, 24)
    m = BlockAllocatorModel(N, B, rng.sample(range(N), N), prefix_caching=True)
    w = PrefixWorld(N, B)
    _random_ops(m, w, rng, 250, alphabet=[0, 1] if seed % 2 else [0, 1, 2], max_prompt=4 * B + 2)
    st = m.cache_stats()
    assert st["hits"] <= st["queries"]


def test_lookup_is_read_only():
    m = BlockAllocatorModel(8, 2, prefix_caching=True)
    m.add_tokens(1, [1, 2, 3, 4, 5])
    m.free_seq(1)
    before = (m.free_list(), m.ref_counts(), dict(m.cache), m.cache_stats())
    assert m.cached_blocks([1, 2, 3, 4]) == m.cached_blocks([1, 2, 3, 4, 9]) != []
    assert (m.free_list(), m.ref_counts(), dict(m.cache), m.cache_stats()) == before


def test_brute_force_short_op_sequences():
    """Every sequence of up to 4 calls drawn from a small menu, B = 2, a pool
    of 3 blocks: the defining property holds after each call."""
    prompts = [[0, 0], [0, 0, 1], [0, 1, 0], [1]]
    menu = [("add", p) for p in range(len(prompts))] + [("append", 0), ("append", 1),
                                                        ("fork",), ("free",)]
    count = 0
    for length in range(1, 5):
        for ops in itertools.product(menu, repeat=length):
            m = BlockAllocatorModel(3, 2, prefix_caching=True)
            w = PrefixWorld(3, 2)
            nid = 0
            for op in ops:
                live = sorted(m.seqs)
                try:
                    if op[0] == "add":
                        toks = prompts[op[1]]
                        slots, cached = m.add_tokens(nid, toks)
                        w.on_add_tokens(nid, toks, slots, cached)
                        nid += 1
                    elif not live:
                        continue
                    elif op[0] == "append":
                        s = live[-1]
                        slot, cow = m.append(s, op[1])
                        if cow:
                            w.on_copy(*cow)
                        w.on_append_token(s, op[1], slot)
                    elif op[0] == "fork":
                        m.fork(live[0], nid)
                        w.on_fork(live[0], nid)
                        nid += 1
                    else:
                        m.free_seq(live[0])
                        w.on_free(live[0])
                except AllocError as e:
                    assert e.code == E_NOBLOCKS
                _check_world(m, w)
                count += 1
    assert count > 1000
