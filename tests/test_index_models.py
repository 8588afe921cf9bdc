"""Host-side models of kernel index arithmetic, checked on the CPU.

decode_partition_mfma_kernel (split-context decode, bf16) stages the table
entries of up to 64 tiles of its partition in LDS and has every wave load its
tiles from there, two tiles ahead, with dead loads (tile -1, or rows past the
partition's end) reading the chunk's last position.  The model below repeats
that index arithmetic and checks that every LDS index lies inside the entries
staged for the chunk, and that the staged count fits the LDS array.
"""

import itertools

import pytest

K_TILE = 16
K_WAVES = 4
K_CHUNK_TILES = 64


def _lds_indices(n, ps, B, p):
    """Yield (index, staged count, array size) for every tile load of partition p."""
    entries = K_CHUNK_TILES * K_TILE // B + 2
    t0 = p * ps
    if t0 >= n:
        return
    t1 = min(n, t0 + ps)
    ntiles = (t1 - t0 + K_TILE - 1) // K_TILE
    for c0 in range(0, ntiles, K_CHUNK_TILES):
        c1 = min(ntiles, c0 + K_CHUNK_TILES)
        cb0 = (t0 + c0 * K_TILE) // B
        cb1 = (min(t1, t0 + c1 * K_TILE) - 1) // B + 1
        last = min(t1, t0 + c1 * K_TILE) - 1
        for wave in range(K_WAVES):
            tile = c0 + wave
            if tile >= c1:
                continue
            mine = (c1 - 1 - tile) // K_WAVES + 1
            loads = [tile]
            for _ in range((mine + 1) // 2):
                tb = tile + K_WAVES
                tc = tile + 2 * K_WAVES
                loads += [tb if tb < c1 else -1, tc if tc < c1 else -1]
                tile += 2 * K_WAVES
            for tl in loads:
                for col in range(16):
                    t = t0 + tl * K_TILE + col
                    live = tl >= 0 and t < t1
                    tok = t if live else last
                    yield tok // B - cb0, cb1 - cb0, entries


@pytest.mark.parametrize("B", [8, 16, 32])
def test_split_context_table_index_stays_in_the_staged_chunk(B):
    lens = [1, B - 1, B, B + 1, 15, 16, 17, 255, 511, 512, 513, 1023, 1024, 1025, 1040, 2047,
            4096, 5000]
    for n, ps in itertools.product(lens, [B, 4 * B, 512, 1024, 2048, None]):
        if ps is None:  # no split: one partition holding the longest context
            ps = -(-n // B) * B
        for p in range(-(-n // ps)):
            for idx, staged, size in _lds_indices(n, ps, B, p):
                assert staged <= size, (n, ps, B, p)
                assert 0 <= idx < staged, (n, ps, B, p, idx, staged)


def test_model_sees_dead_loads():
    # the padded tile loads of a short last chunk are dead and must still be
    # checked (the case the clamp exists for)
    seen_dead = any(True for _ in _lds_indices(40, 512, 16, 0))
    assert seen_dead
