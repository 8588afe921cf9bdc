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


class PrefixWorld(ContentWorld):
    """Slot memory for prefix caching.  A position's K/V depend on every token
    up to it, so each written slot holds the whole token prefix through its
    position, and ``hist[seq][p]`` is the prefix a correct table must show at
    position p.  Positions the allocator reports as already cached are not
    written: they must already hold the right prefix, put there by an earlier
    sequence."""

    def __init__(self, num_blocks: int, block_size: int):
        super().__init__(num_blocks, block_size)
        self.tokens: Dict[int, List[int]] = {}

    def on_add_tokens(self, seq: int, tokens: List[int], slots: List[int], cached: int):
        prefixes = [tuple(tokens[:p + 1]) for p in range(len(tokens))]
        for p in range(cached, len(tokens)):
            self.mem[slots[p]] = prefixes[p]
        self.hist[seq] = prefixes
        self.tokens[seq] = list(tokens)

    def on_fork(self, parent: int, child: int):
        super().on_fork(parent, child)
        self.tokens[child] = list(self.tokens[parent])

    def on_append_token(self, seq: int, token: int, slot: int):
        self.tokens[seq].append(token)
        pre = tuple(self.tokens[seq])
        self.mem[slot] = pre
        self.hist[seq].append(pre)

    def on_free(self, seq: int):
        super().on_free(seq)
        del self.tokens[seq]

    def block_holds(self, block: int, key) -> bool:
        """Block ``block`` holds the K/V of the last full block of prefix ``key``."""
        B = self.B
        i = len(key) // B - 1
        return len(key) % B == 0 and all(
            self.mem.get(block * B + o) == tuple(key[:i * B + o + 1]) for o in range(B))
