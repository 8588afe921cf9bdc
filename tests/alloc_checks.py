"""Semantic checks for a block allocator, independent of how it is written.

An allocator is right when every live sequence reads back its own token
history through its block table, whatever sharing and copying happened on the
way.  ``ContentWorld`` tracks a slot-addressed memory of token ids that is
updated only through what the allocator returns (slots to write, copy pairs
to apply), plus each sequence's history kept on the side; ``check`` compares
the two and checks the bookkeeping invariants.
"""

from __future__ import annotations

import itertools
from typing import Dict, List


class ContentWorld:
    def __init__(self, num_blocks: int, block_size: int):
        self.B = block_size
        self.N = num_blocks
        self.mem: Dict[int, int] = {}
        self.hist: Dict[int, List[int]] = {}
        self._ids = itertools.count(1)

    def fresh(self) -> int:
        return next(self._ids)

    def on_add(self, seq: int, slots: List[int]):
        toks = [self.fresh() for _ in slots]
        for s, t in zip(slots, toks):
            self.mem[s] = t
        self.hist[seq] = toks

    def on_fork(self, parent: int, child: int):
        self.hist[child] = list(self.hist[parent])

    def on_copy(self, src: int, dst: int):
        B = self.B
        for o in range(B):
            if src * B + o in self.mem:
                self.mem[dst * B + o] = self.mem[src * B + o]
            else:
                self.mem.pop(dst * B + o, None)

    def on_append(self, seq: int, slot: int):
        t = self.fresh()
        self.mem[slot] = t
        self.hist[seq].append(t)

    def on_free(self, seq: int):
        del self.hist[seq]


def check(world: ContentWorld, tables: Dict[int, List[int]], lens: Dict[int, int],
          ref: List[int], free: List[int]):
    """tables/lens: live sequences; ref: per-block counts; free: FIFO order."""
    B, N = world.B, world.N
    assert set(tables) == set(world.hist), "live sequence sets differ"
    counted = [0] * N
    for s, t in tables.items():
        n = lens[s]
        assert n == len(world.hist[s])
        assert len(t) == -(-n // B), "a sequence holds exactly ceil(len / B) blocks"
        for b in t:
            assert 0 <= b < N
            counted[b] += 1
        for p in range(n):
            got = world.mem.get(t[p // B] * B + p % B)
            assert got == world.hist[s][p], f"seq {s} position {p} reads {got}"
    assert counted == list(ref), "ref_cnt equals the number of table entries naming the block"
    assert len(set(free)) == len(free)
    used = {b for b in range(N) if ref[b] > 0}
    assert used.isdisjoint(free) and used | set(free) == set(range(N)), \
        "free list and referenced blocks partition the pool"
