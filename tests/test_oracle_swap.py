"""Pins of the oracle's host-pool swapping: a hand-derived trace on the
page's parallel-sampling example, and the defining property -- after any mix
of swaps (whose copy pairs are applied to a device and a host memory), every
sequence reads its own history from the pool it lives in -- plus the
bookkeeping invariants of both pools."""

import random

import pytest

from oracle import AllocError, BlockAllocatorModel, E_INVAL, E_NOBLOCKS
from tests.alloc_checks import ContentWorld


class SwapWorld(ContentWorld):
    """Device slot memory (``mem``) plus host slot memory (``host``)."""

    def __init__(self, num_blocks, block_size):
        super().__init__(num_blocks, block_size)
        self.host = {}

    def on_swap(self, pairs, out: bool):
        B = self.B
        src, dst = (self.mem, self.host) if out else (self.host, self.mem)
        for a, b in pairs:
            for o in range(B):
                if a * B + o in src:
                    dst[b * B + o] = src[a * B + o]
                else:
                    dst.pop(b * B + o, None)


def _check(m: BlockAllocatorModel, w: SwapWorld):
    B = m.block_size
    for pool_seqs, mem, ref, free, N in (
            (m.seqs, w.mem, m.ref, m.free_list(), m.num_blocks),
            (m.swapped, w.host, m.host_ref, m.host_free_list(), len(m.host_ref))):
        counted = [0] * N
        for s, entry in pool_seqs.items():
            table, n = entry[0], entry[1]
            assert len(table) == -(-n // B)
            for b in table:
                counted[b] += 1
            for p in range(n):
                assert mem.get(table[p // B] * B + p % B) == w.hist[s][p], (s, p)
        assert counted == list(ref)
        used = {b for b in range(N) if ref[b] > 0}
        assert len(set(free)) == len(free) and used.isdisjoint(free) and used | set(free) == set(range(N))
    assert set(m.seqs) | set(m.swapped) == set(w.hist) and not set(m.seqs) & set(m.swapped)


def test_hand_derived_trace_on_the_sampling_example():
    m = BlockAllocatorModel(8, 4, [7, 1, 3, 0, 2, 4, 5, 6])
    m.set_host_pool(6)
    m.add(1, 7)                      # A1: [7, 1]
    m.fork(1, 2)                     # A2 shares 7 and 1
    m.append(1)                      # A1 copies block 1 into 3: [7, 3]
    m.append(2)                      # A2 writes block 1 in place: [7, 1]
    pairs = m.swap_out([1, 2])
    assert pairs == [(7, 0), (3, 1), (1, 2)]          # first appearance: 7, 3, then 1
    assert m.free_list() == [0, 2, 4, 5, 6, 1, 3, 7]  # released last pair first
    assert m.host_ref_counts()[:3] == [2, 1, 1]
    assert m.swapped_table(1) == [0, 1] and m.swapped_table(2) == [0, 2]
    pairs = m.swap_in([2, 1])                          # array order decides: A2 first
    assert pairs == [(0, 0), (2, 2), (1, 4)]
    assert m.table(2) == [0, 2] and m.table(1) == [0, 4]
    assert m.host_free_list() == [3, 4, 5, 1, 2, 0]
    assert m.ref_counts()[0] == 2


def test_group_must_own_its_blocks_and_swaps_are_atomic():
    m = BlockAllocatorModel(8, 4)
    m.set_host_pool(2)
    m.add(1, 8)                      # blocks 0, 1
    m.fork(1, 2)
    with pytest.raises(AllocError) as ei:
        m.swap_out([1])              # block 0 and 1 also belong to 2
    assert ei.value.code == E_INVAL
    m.add(3, 12)                     # three blocks, host pool holds two
    before = (m.free_list(), m.ref_counts(), m.host_free_list(), m.host_ref_counts())
    with pytest.raises(AllocError) as ei:
        m.swap_out([3])
    assert ei.value.code == E_NOBLOCKS and ei.value.needed == 3 and ei.value.free == 2
    assert (m.free_list(), m.ref_counts(), m.host_free_list(), m.host_ref_counts()) == before
    assert m.swap_out([1, 2]) == [(0, 0), (1, 1)]
    with pytest.raises(AllocError):
        m.append(1)                  # swapped out: no appends
    m.free_seq(2)
    m.free_seq(1)
    assert sorted(m.host_free_list()) == [0, 1] and m.host_ref_counts() == [0, 0]


def test_swap_without_host_pool_is_rejected():
    m = BlockAllocatorModel(4, 2)
    m.add(1, 3)
    with pytest.raises(AllocError) as ei:
        m.swap_out([1])
    assert ei.value.code == E_INVAL


@pytest.mark.parametrize("seed", range(10))
def test_random_streams_every_sequence_reads_its_history(seed):
    rng = random.Random(seed)
    B = rng.choice([1, 2, 4])
    N, H = rng.randrange(6, 30), rng.randrange(4, 30)
    m = BlockAllocatorModel(N, B, rng.sample(range(N), N))
    m.set_host_pool(H, rng.sample(range(H), H))
    w = SwapWorld(N, B)
    nid = 0
    for _ in range(300):
        live, out = sorted(m.seqs), sorted(m.swapped)
        r = rng.random()
        try:
            if r < 0.2 or not (live or out):
                slots = m.add(nid, rng.randrange(0, 3 * B + 2))
                w.on_add(nid, slots)
                nid += 1
            elif r < 0.3 and live:
                p = rng.choice(live)
                m.fork(p, nid)
                w.on_fork(p, nid)
                nid += 1
            elif r < 0.55 and live:
                seqs = rng.sample(live, rng.randrange(1, len(live) + 1))
                slots, pairs = m.step(seqs)
                for a, b in pairs:
                    w.on_copy(a, b)
                for s, sl in zip(seqs, slots):
                    w.on_append(s, sl)
            elif r < 0.7 and live:
                group = rng.sample(live, rng.randrange(1, len(live) + 1))
                w.on_swap(m.swap_out(group), out=True)
            elif r < 0.85 and out:
                group = rng.sample(out, rng.randrange(1, len(out) + 1))
                w.on_swap(m.swap_in(group), out=False)
            elif live or out:
                s = rng.choice(live + out)
                m.free_seq(s)
                w.on_free(s)
        except AllocError as e:
            assert e.code in (E_INVAL, E_NOBLOCKS)
        _check(m, w)


def test_swapped_ids_stay_taken():
    m = BlockAllocatorModel(8, 2)
    m.set_host_pool(4)
    m.add(1, 3)
    m.swap_out([1])
    for call in (lambda: m.add(1, 1), lambda: m.add_tokens(1, [5]), lambda: m.fork(1, 2)):
        with pytest.raises(AllocError) as ei:
            call()
        assert ei.value.code == E_INVAL
    m.add(2, 1)
    with pytest.raises(AllocError):
        m.fork(2, 1)
