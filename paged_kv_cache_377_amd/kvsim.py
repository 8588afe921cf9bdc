"""KV-cache memory-utilisation simulator: contiguous reservation against paged
blocks, on the host.

What it reproduces is the shape of the pages' argument, not their numbers:
with contiguous KV storage each request must reserve room for the longest
sequence it might reach, so reserved-but-unused slots (reservation waste),
slots never reached (internal fragmentation) and gaps too small for the next
reservation (external fragmentation) leave much of the pool idle; with
fixed-size blocks allocated on demand the only waste is the unfilled tail of
each sequence's last block (zzfmdn.com vLLM article, the paragraphs on the
three kinds of waste and on PagedAttention's blocks; weishuz.com Month 2,
opening paragraph on KV-cache utilisation and section 06 on the block size
trade-off).

Policies (every request r has a prompt of P_r tokens and generates O_r):
  "reserve-max"      reserve max_len contiguous slots at admission
  "reserve-request"  reserve P_r + O_r contiguous slots (an oracle-like
                     scheduler that knows each output length), first fit
  "paged"            the library's block allocator (pkv.BlockAllocator):
                     ceil(P_r / B) blocks at admission, one more block
                     lazily whenever a token crosses into a new block

Scheduler, the same for every policy: time steps; at the start of a step,
waiting requests are admitted first come first served while their admission
fits (a request that does not fit stops admission for the step); then every
running request appends one token; a paged request that cannot get a block
preempts the latest admitted running request (its blocks are freed and it
goes back to the front of the queue to start over, as recomputation);
requests that reach P_r + O_r tokens leave and free their memory.

Per step it records the slots holding tokens, the slots allocated, and the
free slots; the summary gives time-averaged utilisation (stored / pool
capacity, stored / allocated), the reservation and fragmentation shares of
the pool, steps to finish, tokens per step and peak concurrency.
"""

from __future__ import annotations

import bisect
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

E_NOBLOCKS = -2   # the allocators' "not enough free blocks" code


@dataclass
class Request:
    prompt: int
    output: int

    @property
    def total(self) -> int:
        return self.prompt + self.output


def synthetic_requests(n: int, seed: int, max_len: int = 2048, prompt_range=(16, 512),
                       mean_output: float = 256.0) -> List[Request]:
    """Prompts U{16..512}; outputs geometric with the given mean, at least 1,
    capped so that prompt + output <= max_len (most requests end up a few
    hundred tokens long while the reservation is for 2048)."""
    rng = np.random.default_rng(seed)
    prompts = rng.integers(prompt_range[0], prompt_range[1], size=n, endpoint=True)
    outs = rng.geometric(1.0 / mean_output, size=n)
    reqs = []
    for p, o in zip(prompts, outs):
        o = int(min(max(1, o), max_len - int(p)))
        reqs.append(Request(int(p), o))
    return reqs


class FirstFit:
    """Contiguous slot ranges over [0, capacity), first fit by address; free
    ranges are kept sorted and coalesced."""

    def __init__(self, capacity: int):
        self.capacity = capacity
        self.starts: List[int] = [0]
        self.sizes: List[int] = [capacity]

    def alloc(self, size: int) -> Optional[int]:
        for i, sz in enumerate(self.sizes):
            if sz >= size:
                start = self.starts[i]
                if sz == size:
                    del self.starts[i]
                    del self.sizes[i]
                else:
                    self.starts[i] += size
                    self.sizes[i] -= size
                return start
        return None

    def free(self, start: int, size: int) -> None:
        i = bisect.bisect_left(self.starts, start)
        self.starts.insert(i, start)
        self.sizes.insert(i, size)
        # merge with the next, then with the previous range
        if i + 1 < len(self.starts) and self.starts[i] + self.sizes[i] == self.starts[i + 1]:
            self.sizes[i] += self.sizes[i + 1]
            del self.starts[i + 1]
            del self.sizes[i + 1]
        if i > 0 and self.starts[i - 1] + self.sizes[i - 1] == self.starts[i]:
            self.sizes[i - 1] += self.sizes[i]
            del self.starts[i]
            del self.sizes[i]

    def free_slots(self) -> int:
        return sum(self.sizes)

    def largest(self) -> int:
        return max(self.sizes, default=0)


@dataclass
class SimResult:
    policy: str
    capacity: int
    block_size: int
    steps: int = 0
    tokens_generated: int = 0
    preemptions: int = 0
    peak_running: int = 0
    stored: List[int] = field(default_factory=list)      # per step, slots holding tokens
    allocated: List[int] = field(default_factory=list)   # per step, slots owned by requests
    unusable: List[int] = field(default_factory=list)    # per step, free slots in ranges too small
    running: List[int] = field(default_factory=list)
    waiting: List[int] = field(default_factory=list)     # per step, requests still queued

    def summary(self) -> Dict[str, float]:
        st = np.array(self.stored, dtype=np.float64)
        al = np.array(self.allocated, dtype=np.float64)
        un = np.array(self.unusable, dtype=np.float64)
        sat = np.array(self.waiting) > 0
        cap = float(self.capacity)
        busy = al > 0
        return {
            "policy": self.policy,
            "block_size": self.block_size,
            "steps": self.steps,
            "tokens_per_step": self.tokens_generated / max(self.steps, 1),
            "peak_running": self.peak_running,
            "mean_running": float(np.mean(self.running)) if self.running else 0.0,
            "preemptions": self.preemptions,
            "pool_utilisation": float(st.mean() / cap) if len(st) else 0.0,
            "allocated_utilisation": float((st[busy] / al[busy]).mean()) if busy.any() else 0.0,
            "waste_in_allocations": float(((al - st) / cap).mean()) if len(st) else 0.0,
            "external_fragmentation": float((un / cap).mean()) if len(un) else 0.0,
            # while requests are queued the pool is the limit: the share of it
            # holding tokens then is the utilisation the pages compare
            "saturated_steps": int(sat.sum()),
            "saturated_pool_utilisation": float(st[sat].mean() / cap) if sat.any() else 0.0,
            "saturated_running": float(np.array(self.running)[sat].mean()) if sat.any() else 0.0,
        }


def simulate(requests: Sequence[Request], capacity_slots: int, policy: str, max_len: int = 2048,
             block_size: int = 16, allocator_factory: Optional[Callable] = None,
             max_steps: int = 1_000_000) -> SimResult:
    """Run the scheduler over ``requests`` with a pool of ``capacity_slots``
    token slots.  ``allocator_factory(num_blocks, block_size)`` builds the
    paged allocator (default: the library's); it needs add / step / free."""
    if policy not in ("reserve-max", "reserve-request", "paged"):
        raise ValueError(f"unknown policy {policy!r}")
    for r in requests:
        if r.total > max_len or r.prompt < 1 or r.output < 1:
            raise ValueError("every request needs 1 <= prompt, 1 <= output, total <= max_len")
    B = block_size if policy == "paged" else 1
    res = SimResult(policy, capacity_slots, B)
    waiting: List[int] = list(range(len(requests)))
    running: List[int] = []          # admission order
    length: Dict[int, int] = {}
    where: Dict[int, Tuple[int, int]] = {}
    if policy == "paged":
        if allocator_factory is None:
            from ._lib import BlockAllocator
            allocator_factory = BlockAllocator
        nblocks = capacity_slots // B
        alloc = allocator_factory(nblocks, B)
        res.capacity = nblocks * B
        owned: Dict[int, int] = {}
    else:
        ff = FirstFit(capacity_slots)

    def reserve_size(i: int) -> int:
        return max_len if policy == "reserve-max" else requests[i].total

    steps = 0
    while (waiting or running) and steps < max_steps:
        # admission, first come first served
        while waiting:
            i = waiting[0]
            if policy == "paged":
                try:
                    alloc.add(i, requests[i].prompt)
                except Exception as e:       # the allocator's "no blocks" error
                    if getattr(e, "code", None) != E_NOBLOCKS:
                        raise
                    break
                owned[i] = -(-requests[i].prompt // B)
            else:
                start = ff.alloc(reserve_size(i))
                if start is None:
                    break
                where[i] = (start, reserve_size(i))
            waiting.pop(0)
            running.append(i)
            length[i] = requests[i].prompt
        if not running:
            raise ValueError(f"request {waiting[0]} does not fit in an empty pool")
        res.peak_running = max(res.peak_running, len(running))
        # one token per running request
        if policy == "paged":
            k = 0
            while k < len(running):
                i = running[k]
                try:
                    alloc.step([i])
                except Exception as e:       # no free block: preempt the latest admitted
                    if getattr(e, "code", None) != E_NOBLOCKS:
                        raise
                    victim = running.pop()
                    alloc.free(victim)
                    owned.pop(victim)
                    length.pop(victim)
                    waiting.insert(0, victim)
                    res.preemptions += 1
                    continue
                length[i] += 1
                if (length[i] - 1) % B == 0:
                    owned[i] += 1
                res.tokens_generated += 1
                k += 1
        else:
            for i in running:
                length[i] += 1
                res.tokens_generated += 1
        steps += 1
        stored = sum(length[i] for i in running)
        if policy == "paged":
            allocated = sum(owned[i] for i in running) * B
            unusable = 0
        else:
            allocated = sum(where[i][1] for i in running)
            need_next = reserve_size(waiting[0]) if waiting else 0
            unusable = sum(sz for sz in ff.sizes if sz < need_next) if waiting else 0
        res.stored.append(stored)
        res.allocated.append(allocated)
        res.unusable.append(unusable)
        res.running.append(len(running))
        res.waiting.append(len(waiting))
        # departures
        done = [i for i in running if length[i] >= requests[i].total]
        for i in done:
            running.remove(i)
            if policy == "paged":
                alloc.free(i)
                owned.pop(i)
            else:
                ff.free(*where.pop(i))
            length.pop(i)
    res.steps = steps
    return res


def block_size_tradeoff(requests: Sequence[Request], sizes=(1, 2, 4, 8, 16, 32, 64, 128, 256),
                        kv_bytes_per_token: int = 4096, entry_bytes: int = 4) -> List[Dict[str, float]]:
    """For the final lengths L_r of the requests: the unfilled share of the
    last blocks (internal fragmentation, sum (B ceil(L/B) - L) / sum B ceil(L/B))
    against the block table's size relative to the K/V it maps (one entry per
    B tokens of kv_bytes_per_token bytes each)."""
    L = np.array([r.total for r in requests], dtype=np.int64)
    out = []
    for B in sizes:
        slots = B * ((L + B - 1) // B)
        out.append({"block_size": B,
                    "internal_fragmentation": float((slots - L).sum() / slots.sum()),
                    "table_bytes_per_kv_byte": entry_bytes / (B * kv_bytes_per_token),
                    "table_entries": int(((L + B - 1) // B).sum())})
    return out


def main(argv=None) -> None:
    """python -m paged_kv_cache_377_amd.kvsim [--requests N] [--pool-seqs K]
    [--seed S]: the three policies on synthetic requests (max_len 2048, a
    pool of K x 2048 slots) and the block-size trade-off, as JSON lines."""
    import argparse
    import json

    ap = argparse.ArgumentParser()
    ap.add_argument("--requests", type=int, default=1000)
    ap.add_argument("--pool-seqs", type=int, default=16)
    ap.add_argument("--seed", type=int, default=6)
    ap.add_argument("--block-size", type=int, default=16)
    a = ap.parse_args(argv)
    reqs = synthetic_requests(a.requests, a.seed)
    for pol in ("reserve-max", "reserve-request", "paged"):
        r = simulate(reqs, a.pool_seqs * 2048, pol, block_size=a.block_size)
        print(json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.summary().items()}))
    for row in block_size_tradeoff(reqs):
        print(json.dumps({k: (round(v, 6) if isinstance(v, float) else v) for k, v in row.items()}))


if __name__ == "__main__":
    main()
