"""Block-pool model: free list, reference counts, lazy allocation, copy-on-write.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Pure Python, no numpy.

What the pages fix, and where:

* The KV cache of a request is cut into fixed-size logical blocks; each
  sequence owns a block table mapping logical block i to a physical block,
  and a physical block records how many of its slots are filled (page 1,
  section 3(3), step 1) "Prefill": a 7-token prompt with B = 4 takes logical
  blocks 0 and 1, mapped to physical blocks 7 and 1, filled 4 and 3).
* A new physical block is taken only when a new token crosses into the next
  block: allocation is lazy, the analogue of a page fault (page 3, section 02,
  the OS-to-vLLM table, row "page fault").  Page 1, step 2) "Decode" can be
  read as opening block 2 as soon as block 1 fills; this model follows page 3:
  the token that fills a block allocates nothing, the next one opens a block.
* Physical blocks are shared: each carries a reference count, the number of
  logical blocks mapped onto it (page 1, section 4, step (1): samples A1 and A2
  of one prompt share physical blocks 7 and 1, ref count 2).
* When a sample writes its own token into a shared block, that block is copied
  first: the writer gets a fresh block, the shared block's count drops by one
  and the fresh block's count is 1 (page 1, section 4, step (2): A1 writes
  "fathers", gets block 3; block 1 stays with A2).
* The pool keeps an explicit free list of physical blocks and a ``ref_cnt`` per
  block (page 3, section 03, reading (2) on the block pool, and section 04 on
  reference counting); ``allocate_slots()`` / ``free()`` are the manager's
  verbs (page 3, section 03, reading (1)).

Readings taken where the pages are silent:

* The free list is a FIFO: blocks are taken from its head and freed blocks go
  to its tail.  Its initial order is a parameter (default ascending ids).
* A sequence's blocks are released tail-first (deepest logical block first).
* In a batch step the sequences append in array order; the first writer into a
  shared, partially filled block copies it, and the last remaining sharer
  writes in place once the count has fallen to 1.  A shared block that is full
  is never copied: the next token opens a fresh block lazily.
* A batch step is all-or-nothing: if the pool cannot supply every block the
  step needs, nothing changes.  A step may not name one sequence twice.
* Slot of position p in a sequence = table[p // B] * B + p % B.
"""

from __future__ import annotations

from collections import deque
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

E_INVAL = -1
E_NOBLOCKS = -2


class AllocError(Exception):
    """An allocator call that failed and left the state unchanged."""

    def __init__(self, code: int, message: str, needed: int = 0, free: int = 0,
                 total: int = 0):
        super().__init__(message)
        self.code = code
        self.needed = needed
        self.free = free
        self.total = total


class BlockAllocatorModel:
    """Reference model of the host block allocator."""

    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise AllocError(E_INVAL, "num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocError(E_INVAL, "free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: deque = deque(order)
        self.ref: List[int] = [0] * num_blocks
        # seq id -> [block table (list of physical ids), number of tokens]
        self.seqs: Dict[int, list] = {}

    # ------------------------------------------------------------------ helpers
    def _no_blocks(self, needed: int) -> AllocError:
        free = len(self.free)
        return AllocError(
            E_NOBLOCKS,
            f"failed to allocate {needed} blocks: {free} free of {self.num_blocks} total",
            needed, free, self.num_blocks)

    def _take(self) -> int:
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def _slot(self, table: List[int], pos: int) -> int:
        B = self.block_size
        return table[pos // B] * B + pos % B

    # ------------------------------------------------------------------ verbs
    def add(self, seq: int, num_tokens: int) -> List[int]:
        """Admit a sequence holding ``num_tokens`` tokens (the prompt).

        Takes ceil(n / B) blocks from the head of the free list and returns the
        slot of every prompt position (page 1, section 3(3), step 1)).
        """
        if seq in self.seqs or num_tokens < 0:
            raise AllocError(E_INVAL, f"bad add of sequence {seq}")
        B = self.block_size
        needed = -(-num_tokens // B)
        if needed > len(self.free):
            raise self._no_blocks(needed)
        table = [self._take() for _ in range(needed)]
        self.seqs[seq] = [table, num_tokens]
        return [self._slot(table, p) for p in range(num_tokens)]

    def fork(self, parent: int, child: int) -> None:
        """``child`` starts as a copy of ``parent``'s table; every block gains a
        reference (page 1, section 4, step (1))."""
        if parent not in self.seqs or child in self.seqs:
            raise AllocError(E_INVAL, f"bad fork {parent} -> {child}")
        table, length = self.seqs[parent]
        for b in table:
            self.ref[b] += 1
        self.seqs[child] = [list(table), length]

    def append(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot for one new token of ``seq``.

        Returns (slot, cow) where cow is (src, dst) when the shared last block
        had to be copied before this token is written into it, else None.
        """
        if seq not in self.seqs:
            raise AllocError(E_INVAL, f"unknown sequence {seq}")
        table, pos = self.seqs[seq]
        B = self.block_size
        cow = None
        if pos % B == 0:
            # The new token crosses into a block not yet mapped: lazy allocation.
            if not self.free:
                raise self._no_blocks(1)
            table.append(self._take())
        else:
            last = table[pos // B]
            if self.ref[last] > 1:
                # Divergent write into a shared, partially filled block.
                if not self.free:
                    raise self._no_blocks(1)
                fresh = self._take()
                self.ref[last] -= 1
                table[pos // B] = fresh
                cow = (last, fresh)
        slot = self._slot(table, pos)
        self.seqs[seq][1] = pos + 1
        return slot, cow

    def step(self, seqs: Iterable[int]) -> Tuple[List[int], List[Tuple[int, int]]]:
        """One decode step: append one token to each sequence, in array order.

        All-or-nothing: the blocks the whole step takes are counted first, and
        if the pool holds fewer nothing changes.  For ``E_NOBLOCKS`` the message
        names that count, the free count and the pool size.
        """
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs) or any(s not in self.seqs for s in seqs):
            raise AllocError(E_INVAL, "step names an unknown or repeated sequence")
        B = self.block_size
        ref = list(self.ref)
        needed = 0
        for s in seqs:
            table, pos = self.seqs[s]
            if pos % B == 0:
                needed += 1
            elif ref[table[pos // B]] > 1:
                needed += 1
                ref[table[pos // B]] -= 1
        if needed > len(self.free):
            raise self._no_blocks(needed)
        slots: List[int] = []
        pairs: List[Tuple[int, int]] = []
        for s in seqs:
            slot, cow = self.append(s)
            slots.append(slot)
            if cow is not None:
                pairs.append(cow)
        return slots, pairs

    def free_seq(self, seq: int) -> None:
        """Release a finished sequence: walk its table from the last block to
        the first; a block whose count reaches 0 goes to the free-list tail."""
        if seq not in self.seqs:
            raise AllocError(E_INVAL, f"unknown sequence {seq}")
        table, _ = self.seqs.pop(seq)
        for b in reversed(table):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    # ------------------------------------------------------------------ views
    def table(self, seq: int) -> List[int]:
        return list(self.seqs[seq][0])

    def length(self, seq: int) -> int:
        return self.seqs[seq][1]

    def filled(self, seq: int) -> List[int]:
        """'# filled' of each of the sequence's blocks (page 1, section 3(3))."""
        table, n = self.seqs[seq]
        B = self.block_size
        return [min(B, n - i * B) for i in range(len(table))]

    def build_tables(self, seqs: Sequence[int], width: int,
                     pad: int = 0) -> Tuple[List[List[int]], List[int]]:
        """Block tables padded to ``width`` entries, plus context lengths."""
        tables, lens = [], []
        for s in seqs:
            if s not in self.seqs:
                raise AllocError(E_INVAL, f"unknown sequence {s}")
            t, n = self.seqs[s]
            if len(t) > width:
                raise AllocError(E_INVAL, f"sequence {s} holds {len(t)} blocks > width {width}")
            tables.append(list(t) + [pad] * (width - len(t)))
            lens.append(n)
        return tables, lens

    def free_list(self) -> List[int]:
        return list(self.free)

    def ref_counts(self) -> List[int]:
        return list(self.ref)
