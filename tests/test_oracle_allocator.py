"""Pins of the oracle's allocator model against what the pages print and what
the semantics force (every sequence reads back its own history)."""

import copy
import json
import os
import random

import pytest

from oracle import AllocError, BlockAllocatorModel, E_INVAL, E_NOBLOCKS
from tests.alloc_checks import ContentWorld, check


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _refs(model, keys):
    return {str(k): model.ref_counts()[int(k)] for k in keys}


def test_toy_prefill_decode_trace(golden_dir):
    g = _load(golden_dir, "toy_prefill_decode_trace.json")
    m = BlockAllocatorModel(g["num_blocks"], g["block_size"], g["free_order"])
    for op in g["ops"]:
        e = op["expect"]
        if op["op"] == "add":
            slots = m.add(op["seq"], op["num_tokens"])
            assert slots == e["slots"]
        else:
            slot, cow = m.append(op["seq"])
            assert slot == e["slot"]
            assert cow == (None if e["cow"] is None else tuple(e["cow"]))
        assert m.table(op["seq"]) == e["table"]
        assert m.filled(op["seq"]) == e["filled"]
    assert _refs(m, g["final"]["ref_cnt"]) == g["final"]["ref_cnt"]
    assert m.free_list() == g["final"]["free"]


def test_parallel_sampling_cow_trace(golden_dir):
    g = _load(golden_dir, "parallel_sampling_cow_trace.json")
    m = BlockAllocatorModel(g["num_blocks"], g["block_size"], g["free_order"])
    B = g["block_size"]
    words = {}          # slot -> word, the "physical memory" of the example
    history = {}
    for op in g["ops"]:
        e = op["expect"]
        if op["op"] == "add":
            slots = m.add(op["seq"], op["num_tokens"])
            assert slots == e["slots"]
            for s, w in zip(slots, g["prompt"]):
                words[s] = w
            history[op["seq"]] = list(g["prompt"])
            assert m.filled(op["seq"]) == e["filled"]
        elif op["op"] == "fork":
            m.fork(op["parent"], op["child"])
            history[op["child"]] = list(history[op["parent"]])
            assert _refs(m, e["ref_cnt"]) == e["ref_cnt"]
            for s, t in e["tables"].items():
                assert m.table(int(s)) == t
        else:
            slot, cow = m.append(op["seq"])
            assert slot == e["slot"]
            assert cow == (None if e["cow"] is None else tuple(e["cow"]))
            if cow is not None:
                src, dst = cow
                for o in range(B):
                    if src * B + o in words:
                        words[dst * B + o] = words[src * B + o]
            words[slot] = op["token"]
            history[op["seq"]].append(op["token"])
            assert m.table(op["seq"]) == e["table"]
            assert _refs(m, e["ref_cnt"]) == e["ref_cnt"]
    f = g["final"]
    assert _refs(m, f["ref_cnt"]) == f["ref_cnt"]
    assert m.free_list() == f["free"]
    for s, ws in f["sequence_words"].items():
        t = m.table(int(s))
        got = [words[t[p // B] * B + p % B] for p in range(m.length(int(s)))]
        assert got == ws == history[int(s)]
    for b, ws in f["block_words"].items():
        assert [words[int(b) * B + o] for o in range(B)] == ws


def _state(m):
    return (m.free_list(), m.ref_counts(),
            {s: (m.table(s), m.length(s)) for s in m.seqs})


def _world_check(world, m):
    check(world, {s: m.table(s) for s in m.seqs}, {s: m.length(s) for s in m.seqs},
          m.ref_counts(), m.free_list())


def _apply(m, world, op):
    """Apply one op to model and world; return True if it succeeded.  A failed
    op must leave the model unchanged."""
    before = _state(m)
    kind = op[0]
    try:
        if kind == "add":
            slots = m.add(op[1], op[2])
            world.on_add(op[1], slots)
        elif kind == "fork":
            m.fork(op[1], op[2])
            world.on_fork(op[1], op[2])
        elif kind == "append":
            slot, cow = m.append(op[1])
            if cow is not None:
                world.on_copy(*cow)
            world.on_append(op[1], slot)
        elif kind == "step":
            slots, pairs = m.step(op[1])
            # all copies are applied before any token is written
            for src, dst in pairs:
                world.on_copy(src, dst)
            for s, sl in zip(op[1], slots):
                world.on_append(s, sl)
        elif kind == "free":
            m.free_seq(op[1])
            world.on_free(op[1])
        return True
    except AllocError as e:
        assert e.code in (E_INVAL, E_NOBLOCKS)
        assert _state(m) == before, "a failed call must not change the state"
        return False


def test_step_copies_before_any_write():
    # A step whose copy source is a block another sequence in the same step
    # writes into: A and B share a partial block; the step appends A then B.
    m = BlockAllocatorModel(4, 4)
    w = ContentWorld(4, 4)
    assert _apply(m, w, ("add", 0, 2))
    assert _apply(m, w, ("fork", 0, 1))
    assert _apply(m, w, ("step", [0, 1]))
    _world_check(w, m)
    assert m.table(0) != m.table(1)


def test_lazy_allocation_block_count():
    m = BlockAllocatorModel(16, 4)
    m.add(0, 0)
    assert m.table(0) == []
    for n in range(1, 30):
        m.append(0)
        assert len(m.table(0)) == -(-n // 4)


def test_no_blocks_message_and_atomicity():
    m = BlockAllocatorModel(3, 2)
    m.add(0, 4)          # takes 2 blocks
    m.add(1, 0)
    m.append(1)          # takes the last block
    before = _state(m)
    with pytest.raises(AllocError) as ei:
        m.step([1, 0])   # seq 1 fits in place, seq 0 needs a new block
    assert ei.value.code == E_NOBLOCKS
    assert str(ei.value) == "failed to allocate 1 blocks: 0 free of 3 total"
    assert _state(m) == before
    with pytest.raises(AllocError) as ei:
        m.step([0, 0])
    assert ei.value.code == E_INVAL


OPS_SMALL = [("add", 0, 0), ("add", 0, 1), ("add", 0, 3), ("add", 1, 2),
             ("fork", 0, 1), ("fork", 1, 0), ("append", 0), ("append", 1),
             ("step", [0, 1]), ("step", [1, 0]), ("free", 0), ("free", 1)]


def test_brute_force_all_short_op_sequences():
    """Every sequence of up to 4 ops from OPS_SMALL on a 3-block pool, B = 2."""
    count = 0

    def dfs(m, w, depth):
        nonlocal count
        count += 1
        _world_check(w, m)
        if depth == 4:
            return
        for op in OPS_SMALL:
            m2, w2 = copy.deepcopy(m), copy.deepcopy(w)
            _apply(m2, w2, op)
            dfs(m2, w2, depth + 1)

    dfs(BlockAllocatorModel(3, 2, [2, 0, 1]), ContentWorld(3, 2), 0)
    assert count == sum(len(OPS_SMALL) ** k for k in range(5))


@pytest.mark.parametrize("seed", range(6))
def test_random_op_streams(seed):
    rnd = random.Random(seed)
    B = rnd.choice([1, 2, 4, 8, 16])
    N = rnd.choice([4, 8, 16, 64])
    order = list(range(N))
    rnd.shuffle(order)
    m = BlockAllocatorModel(N, B, order)
    w = ContentWorld(N, B)
    ids = list(range(8))
    ok = 0
    for _ in range(400):
        r = rnd.random()
        live = list(m.seqs)
        if r < 0.15:
            ok += _apply(m, w, ("add", rnd.choice(ids), rnd.randint(0, 3 * B)))
        elif r < 0.25 and live:
            ok += _apply(m, w, ("fork", rnd.choice(live), rnd.choice(ids)))
        elif r < 0.5 and live:
            ok += _apply(m, w, ("append", rnd.choice(live)))
        elif r < 0.85 and live:
            k = rnd.randint(1, len(live))
            ok += _apply(m, w, ("step", rnd.sample(live, k)))
        elif live:
            ok += _apply(m, w, ("free", rnd.choice(live)))
        _world_check(w, m)
    assert ok > 100


def test_rejects_bad_arguments():
    m = BlockAllocatorModel(4, 2)
    m.add(0, 1)
    for op in [lambda: m.add(0, 1), lambda: m.add(1, -1), lambda: m.fork(5, 6),
               lambda: m.fork(0, 0), lambda: m.append(9), lambda: m.free_seq(9),
               lambda: m.build_tables([0], 0)]:
        with pytest.raises(AllocError) as ei:
            op()
        assert ei.value.code == E_INVAL
    with pytest.raises(AllocError):
        BlockAllocatorModel(4, 2, [0, 1, 1, 2])


def test_free_list_order_reading(golden_dir):
    g = _load(golden_dir, "free_list_reading.json")
    m = BlockAllocatorModel(g["num_blocks"], g["block_size"], g["free_order"])
    for op in g["ops"]:
        if op["op"] == "add":
            m.add(op["seq"], op["num_tokens"])
            assert m.table(op["seq"]) == op["expect_table"]
        elif op["op"] == "fork":
            m.fork(op["parent"], op["child"])
        else:
            m.free_seq(op["seq"])
            assert m.free_list() == op["expect_free"]
