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

Prefix caching (optional, ``prefix_caching=True``), after page 3, section 04
and section 03 reading (2):

* A full block whose tokens are known is entered in a map from its key to its
  physical block once the tokens that fill it have been given a slot; a later
  prompt whose leading full blocks have the same keys maps those blocks
  instead of computing them again (the page's two requests share a 16-token
  system prompt: the second finds the first one's block and skips its
  prefill).  The key of logical block i is the whole token prefix through the
  end of block i, so two blocks share a key only when everything before them
  matched too: the prefix-aware chain the page asks for, here without any
  hash, hence without collisions.
* Blocks stay in the map after their count drops to 0: they wait in the free
  list, in release order, and a hit takes such a block back out of the list.
  A block is evicted (leaves the map) only when the free list hands it out
  again, so the least recently released block goes first, and a referenced
  block is never evicted (page 3, section 04: evict under memory pressure,
  LRU, never a referenced block).

Readings taken where the pages are silent:

* A prompt's lookup walks its full blocks from the first and stops at the
  first miss; a prompt's partial last block is never looked up.
* A prompt first takes back its hit blocks (those with count 0 leave the free
  list), then takes fresh blocks from the free-list head, and then enters its
  full, missed blocks in the map.  Blocks filled later by single appends are
  entered when their last slot is handed out.
* If a key is already in the map, the first block entered keeps it; the new
  block stays out of the map.
* A sequence keeps its token history only while every token it was given
  came with an id; after an append without one, none of its later blocks is
  entered.  A fork copies the parent's history.
* Cache statistics count every full prompt block looked up (a query) and
  every block found (a hit); the hit rate is hits / queries.

Swapping (optional host pool; page 3, section 02, the OS-to-vLLM table, row
"swap to disk": blocks of preempted requests move to host memory and back):

* A group of sequences moves as a whole.  Every block they map is copied
  once (first appearance in array order, then table order) to a host block
  taken from the host free list's head; the copy pairs are returned in that
  order, the host block inherits the device block's count, and the device
  blocks are then released last pair first (as a finished sequence releases
  its blocks).  Swapping in is the mirror image.
* Readings: a block the group shares with a sequence outside it cannot move
  (E_INVAL); a swap is all-or-nothing (E_NOBLOCKS when the target pool holds
  fewer free blocks than the group's distinct blocks); a swapped-out
  sequence cannot append, fork or be tabled until it is swapped back in, but
  it can be freed (its host blocks go to the host free list's tail).
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
                 free_order: Optional[Sequence[int]] = None,
                 prefix_caching: bool = False):
        if num_blocks <= 0 or block_size <= 0:
            raise AllocError(E_INVAL, "num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocError(E_INVAL, "free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: deque = deque(order)
        self.ref: List[int] = [0] * num_blocks
        # seq id -> [block table (list of physical ids), number of tokens,
        #            token history (list of ids) or None when unknown]
        self.seqs: Dict[int, list] = {}
        self.prefix_caching = bool(prefix_caching)
        self.cache: Dict[Tuple[int, ...], int] = {}   # prefix key -> block
        self.block_key: Dict[int, Tuple[int, ...]] = {}
        self.hits = 0
        self.queries = 0
        self.evictions = 0
        # host pool for swapped-out sequences (empty until set_host_pool)
        self.host_free: deque = deque()
        self.host_ref: List[int] = []
        self.swapped: Dict[int, list] = {}

    # ------------------------------------------------------------------ helpers
    def _no_blocks(self, needed: int) -> AllocError:
        free = len(self.free)
        return AllocError(
            E_NOBLOCKS,
            f"failed to allocate {needed} blocks: {free} free of {self.num_blocks} total",
            needed, free, self.num_blocks)

    def _take(self) -> int:
        b = self.free.popleft()
        key = self.block_key.pop(b, None)
        if key is not None:          # the cached contents are about to be overwritten
            del self.cache[key]
            self.evictions += 1
        self.ref[b] = 1
        return b

    def _enter(self, block: int, key: Tuple[int, ...]) -> None:
        if self.prefix_caching and key not in self.cache:
            self.cache[key] = block
            self.block_key[block] = key

    def _lookup(self, tokens: Sequence[int]) -> List[int]:
        """Blocks holding the longest run of the prompt's leading full blocks."""
        B = self.block_size
        found: List[int] = []
        for i in range(len(tokens) // B):
            b = self.cache.get(tuple(tokens[:(i + 1) * B]))
            if b is None:
                break
            found.append(b)
        return found

    def _slot(self, table: List[int], pos: int) -> int:
        B = self.block_size
        return table[pos // B] * B + pos % B

    # ------------------------------------------------------------------ verbs
    def add(self, seq: int, num_tokens: int) -> List[int]:
        """Admit a sequence holding ``num_tokens`` tokens (the prompt).

        Takes ceil(n / B) blocks from the head of the free list and returns the
        slot of every prompt position (page 1, section 3(3), step 1)).
        """
        if seq in self.seqs or seq in self.swapped or num_tokens < 0:
            raise AllocError(E_INVAL, f"bad add of sequence {seq}")
        B = self.block_size
        needed = -(-num_tokens // B)
        if needed > len(self.free):
            raise self._no_blocks(needed)
        table = [self._take() for _ in range(needed)]
        self.seqs[seq] = [table, num_tokens, None]
        return [self._slot(table, p) for p in range(num_tokens)]

    def add_tokens(self, seq: int, tokens: Sequence[int]) -> Tuple[List[int], int]:
        """Admit a prompt given by its token ids.

        With prefix caching, the prompt's leading full blocks found in the
        cache are mapped instead of new ones (page 3, section 04).  Returns the
        slot of every prompt position and the number of leading positions
        whose K/V the cache already holds; only the positions after those
        still have to be written.  All-or-nothing: the blocks taken out of the
        free list (fresh ones, plus hits whose count was 0) are counted first.
        """
        tokens = [int(t) for t in tokens]
        if seq in self.seqs or seq in self.swapped:
            raise AllocError(E_INVAL, f"bad add of sequence {seq}")
        B = self.block_size
        n = len(tokens)
        hits = self._lookup(tokens) if self.prefix_caching else []
        fresh = -(-n // B) - len(hits)
        revived = sum(1 for b in hits if self.ref[b] == 0)
        if fresh + revived > len(self.free):
            raise self._no_blocks(fresh + revived)
        if self.prefix_caching:
            self.queries += n // B
            self.hits += len(hits)
        for b in hits:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
        table = hits + [self._take() for _ in range(fresh)]
        for i in range(len(hits), n // B):
            self._enter(table[i], tuple(tokens[:(i + 1) * B]))
        self.seqs[seq] = [table, n, tokens]
        return [self._slot(table, p) for p in range(n)], len(hits) * B

    def cached_blocks(self, tokens: Sequence[int]) -> List[int]:
        """Read-only lookup: the cached blocks a prompt of these tokens would
        map (the manager's get_cached_blocks(), page 3, section 03 reading (1))."""
        return self._lookup([int(t) for t in tokens]) if self.prefix_caching else []

    def cache_stats(self) -> Dict[str, int]:
        return {"hits": self.hits, "queries": self.queries,
                "cached_blocks": len(self.cache), "evictions": self.evictions}

    def fork(self, parent: int, child: int) -> None:
        """``child`` starts as a copy of ``parent``'s table; every block gains a
        reference (page 1, section 4, step (1))."""
        if parent not in self.seqs or child in self.seqs or child in self.swapped:
            raise AllocError(E_INVAL, f"bad fork {parent} -> {child}")
        table, length, toks = self.seqs[parent]
        for b in table:
            self.ref[b] += 1
        self.seqs[child] = [list(table), length, None if toks is None else list(toks)]

    def append(self, seq: int, token: Optional[int] = None) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot for one new token of ``seq``.

        Returns (slot, cow) where cow is (src, dst) when the shared last block
        had to be copied before this token is written into it, else None.
        ``token`` (its id, optional) extends the sequence's history; with
        prefix caching a block this token fills is entered in the cache.
        """
        if seq not in self.seqs:
            raise AllocError(E_INVAL, f"unknown sequence {seq}")
        table, pos, _ = self.seqs[seq]
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
        entry = self.seqs[seq]
        entry[1] = pos + 1
        if token is None:
            entry[2] = None
        elif entry[2] is not None:
            entry[2].append(int(token))
            if (pos + 1) % B == 0:
                self._enter(table[pos // B], tuple(entry[2]))
        return slot, cow

    def step(self, seqs: Iterable[int], tokens: Optional[Sequence[int]] = None
             ) -> Tuple[List[int], List[Tuple[int, int]]]:
        """One decode step: append one token to each sequence, in array order.

        All-or-nothing: the blocks the whole step takes are counted first, and
        if the pool holds fewer nothing changes.  For ``E_NOBLOCKS`` the message
        names that count, the free count and the pool size.  ``tokens``, when
        given, holds the id of each sequence's new token.
        """
        seqs = [int(s) for s in seqs]
        if tokens is not None and len(tokens) != len(seqs):
            raise AllocError(E_INVAL, "step: one token id per sequence")
        if len(set(seqs)) != len(seqs) or any(s not in self.seqs for s in seqs):
            raise AllocError(E_INVAL, "step names an unknown or repeated sequence")
        B = self.block_size
        ref = list(self.ref)
        needed = 0
        for s in seqs:
            table, pos, _ = self.seqs[s]
            if pos % B == 0:
                needed += 1
            elif ref[table[pos // B]] > 1:
                needed += 1
                ref[table[pos // B]] -= 1
        if needed > len(self.free):
            raise self._no_blocks(needed)
        slots: List[int] = []
        pairs: List[Tuple[int, int]] = []
        for j, s in enumerate(seqs):
            slot, cow = self.append(s, None if tokens is None else tokens[j])
            slots.append(slot)
            if cow is not None:
                pairs.append(cow)
        return slots, pairs

    def free_seq(self, seq: int) -> None:
        """Release a finished sequence: walk its table from the last block to
        the first; a block whose count reaches 0 goes to the free-list tail
        (the host pool's, for a swapped-out sequence)."""
        if seq in self.swapped:
            for b in reversed(self.swapped.pop(seq)[0]):
                self.host_ref[b] -= 1
                if self.host_ref[b] == 0:
                    self.host_free.append(b)
            return
        if seq not in self.seqs:
            raise AllocError(E_INVAL, f"unknown sequence {seq}")
        table = self.seqs.pop(seq)[0]
        for b in reversed(table):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    # ------------------------------------------------------------------ swap
    def set_host_pool(self, num_blocks: int, free_order: Optional[Sequence[int]] = None) -> None:
        if self.host_ref or num_blocks <= 0:
            raise AllocError(E_INVAL, "the host pool is set once, with a positive size")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocError(E_INVAL, "host free_order must be a permutation")
        self.host_free = deque(order)
        self.host_ref = [0] * num_blocks

    def _move(self, seqs, src_seqs, dst_seqs, src_ref, dst_ref, dst_take, src_release):
        seqs = [int(x) for x in seqs]
        if len(set(seqs)) != len(seqs) or any(x not in src_seqs for x in seqs):
            raise AllocError(E_INVAL, "swap names an unknown, repeated or misplaced sequence")
        order: List[int] = []
        count: Dict[int, int] = {}
        for x in seqs:
            for b in src_seqs[x][0]:
                if b not in count:
                    count[b] = 0
                    order.append(b)
                count[b] += 1
        for b in order:
            if count[b] != src_ref[b]:
                raise AllocError(E_INVAL, f"block {b} is shared with a sequence outside the group")
        dst_free = self.free if dst_seqs is self.seqs else self.host_free
        if len(order) > len(dst_free):
            free = len(dst_free)
            total = self.num_blocks if dst_seqs is self.seqs else len(self.host_ref)
            raise AllocError(E_NOBLOCKS,
                             f"failed to allocate {len(order)} blocks: {free} free of {total} total",
                             len(order), free, total)
        where: Dict[int, int] = {}
        pairs: List[Tuple[int, int]] = []
        for b in order:
            d = dst_take()
            dst_ref[d] = src_ref[b]
            where[b] = d
            pairs.append((b, d))
        for b, _ in reversed(pairs):
            src_ref[b] = 0
            src_release(b)
        for x in seqs:
            entry = src_seqs.pop(x)
            entry[0] = [where[b] for b in entry[0]]
            dst_seqs[x] = entry
        return pairs

    def swap_out(self, seqs: Iterable[int]) -> List[Tuple[int, int]]:
        """Move a group of sequences to the host pool; returns (device block,
        host block) copy pairs.  The caller copies them before reusing the
        released device blocks."""
        if not self.host_ref:
            raise AllocError(E_INVAL, "no host pool")

        def take_host():
            return self.host_free.popleft()

        return self._move(seqs, self.seqs, self.swapped, self.ref, self.host_ref, take_host,
                          self.free.append)

    def swap_in(self, seqs: Iterable[int]) -> List[Tuple[int, int]]:
        """Move a group of swapped-out sequences back; returns (host block,
        device block) copy pairs, to be copied before the group is used."""
        return self._move(seqs, self.swapped, self.seqs, self.host_ref, self.ref, self._take,
                          self.host_free.append)

    def host_free_list(self) -> List[int]:
        return list(self.host_free)

    def host_ref_counts(self) -> List[int]:
        return list(self.host_ref)

    def swapped_table(self, seq: int) -> List[int]:
        return list(self.swapped[seq][0])

    # ------------------------------------------------------------------ views
    def table(self, seq: int) -> List[int]:
        return list(self.seqs[seq][0])

    def length(self, seq: int) -> int:
        return self.seqs[seq][1]

    def filled(self, seq: int) -> List[int]:
        """'# filled' of each of the sequence's blocks (page 1, section 3(3))."""
        table, n = self.seqs[seq][:2]
        B = self.block_size
        return [min(B, n - i * B) for i in range(len(table))]

    def build_tables(self, seqs: Sequence[int], width: int,
                     pad: int = 0) -> Tuple[List[List[int]], List[int]]:
        """Block tables padded to ``width`` entries, plus context lengths."""
        tables, lens = [], []
        for s in seqs:
            if s not in self.seqs:
                raise AllocError(E_INVAL, f"unknown sequence {s}")
            t, n = self.seqs[s][:2]
            if len(t) > width:
                raise AllocError(E_INVAL, f"sequence {s} holds {len(t)} blocks > width {width}")
            tables.append(list(t) + [pad] * (width - len(t)))
            lens.append(n)
        return tables, lens

    def free_list(self) -> List[int]:
        return list(self.free)

    def ref_counts(self) -> List[int]:
        return list(self.ref)
