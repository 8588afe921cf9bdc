"""Pins of the oracle's slot_mapping write and block copy."""

import numpy as np

from datagen import BF16_NAN, bf16_from_f32
from oracle import BlockAllocatorModel, copy_blocks, paged_kv_write


def _pool(rng, nb, h, b, d, dtype):
    if dtype == "bf16":
        return bf16_from_f32(rng.standard_normal((nb, h, b, d)).astype(np.float32))
    return rng.standard_normal((nb, h, b, d)).astype(np.float32)


def test_write_touches_exactly_the_named_slots():
    rng = np.random.default_rng(7)
    nb, h, B, d = 6, 3, 4, 5
    for dtype in ("bf16", "f32"):
        kc, vc = _pool(rng, nb, h, B, d, dtype), _pool(rng, nb, h, B, d, dtype)
        slots = np.array([5, -1, 0, 23, nb * B, 17, 2 ** 40, 9], dtype=np.int64)
        T = len(slots)
        k, v = _pool(rng, T, h, 1, d, dtype)[:, :, 0], _pool(rng, T, h, 1, d, dtype)[:, :, 0]
        kc2, vc2 = paged_kv_write(k, v, slots, kc, vc)
        touched = np.zeros((nb, B), dtype=bool)
        for t, s in enumerate(slots):
            if 0 <= s < nb * B:
                touched[s // B, s % B] = True
                # reading the slot back gives the token's bits, for every head
                assert kc2.view(np.uint8)[s // B, :, s % B].tobytes() == k.view(np.uint8)[t].tobytes()
                assert vc2.view(np.uint8)[s // B, :, s % B].tobytes() == v.view(np.uint8)[t].tobytes()
        assert touched.sum() == 5
        for b in range(nb):
            for o in range(B):
                if not touched[b, o]:
                    assert np.array_equal(kc2[b, :, o].view(np.uint8), kc[b, :, o].view(np.uint8))
                    assert np.array_equal(vc2[b, :, o].view(np.uint8), vc[b, :, o].view(np.uint8))
        # inputs are not modified
        assert kc2 is not kc


def test_copy_blocks_snapshot_and_bits():
    rng = np.random.default_rng(8)
    nb, h, B, d = 8, 2, 4, 3
    kc = bf16_from_f32(rng.standard_normal((nb, h, B, d)).astype(np.float32))
    vc = bf16_from_f32(rng.standard_normal((nb, h, B, d)).astype(np.float32))
    kc[1, 0, 2, 1] = BF16_NAN          # NaN payloads copy bit for bit
    vc[1, 1, 3, 0] = np.uint16(0xFF81)  # a signalling-NaN pattern
    pairs = [(1, 3), (1, 5), (2, 6)]    # one source, several destinations
    kc2, vc2 = copy_blocks(kc, vc, pairs)
    for s, dd in pairs:
        assert np.array_equal(kc2[dd], kc[s]) and np.array_equal(vc2[dd], vc[s])
    for b in (0, 1, 2, 4, 7):
        assert np.array_equal(kc2[b], kc[b]) and np.array_equal(vc2[b], vc[b])


def test_copy_blocks_reads_sources_as_before_the_call():
    """The oracle's copy is a batch: a destination takes its source's contents
    from before the call even when an earlier pair wrote that source (the
    library's contract excludes such chains, and pkv_validate_copy refuses
    them; this pins only the oracle's own definition)."""
    rng = np.random.default_rng(9)
    kc = bf16_from_f32(rng.standard_normal((6, 2, 4, 3)).astype(np.float32))
    vc = bf16_from_f32(rng.standard_normal((6, 2, 4, 3)).astype(np.float32))
    kc2, vc2 = copy_blocks(kc, vc, [(1, 3), (3, 5)])
    assert np.array_equal(kc2[3], kc[1]) and np.array_equal(vc2[3], vc[1])
    assert np.array_equal(kc2[5], kc[3]) and np.array_equal(vc2[5], vc[3])
    assert not np.array_equal(kc[3], kc[1])


def test_cow_flow_carries_prefix_before_divergent_write():
    """Page 1 section 4: the copy carries the shared prefix into the fresh
    block, then the divergent token lands in it; the sibling is untouched."""
    B, h, d = 4, 1, 2
    m = BlockAllocatorModel(8, B, [7, 1, 3, 0, 2, 4, 5, 6])
    kc = np.zeros((8, h, B, d), dtype=np.float32)
    vc = np.zeros_like(kc)
    prompt = np.arange(1, 8, dtype=np.float32)[:, None, None] * np.ones((1, h, d), np.float32)
    kc, vc = paged_kv_write(prompt, -prompt, m.add(1, 7), kc, vc)
    m.fork(1, 2)
    slots, pairs = m.step([1, 2])
    assert pairs == [(1, 3)] and slots == [15, 7]
    kc, vc = copy_blocks(kc, vc, pairs)
    new = np.array([100.0, 200.0], dtype=np.float32)[:, None, None] * np.ones((1, h, d), np.float32)
    kc, vc = paged_kv_write(new, -new, slots, kc, vc)
    assert kc[3, 0, :, 0].tolist() == [5.0, 6.0, 7.0, 100.0]
    assert kc[1, 0, :, 0].tolist() == [5.0, 6.0, 7.0, 200.0]
    assert vc[3, 0, :, 0].tolist() == [-5.0, -6.0, -7.0, -100.0]
