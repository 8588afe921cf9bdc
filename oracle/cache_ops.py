"""slot_mapping write and block copy, on raw bit patterns.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Cache layout: ``k_cache`` and ``v_cache`` are ``[num_blocks, num_kv_heads,
block_size, head_dim]``; physical block b, head h, in-block offset o, lane d.
Both functions work on any element type (they move bits, never values), so
``uint16`` bf16 bit arrays and ``float32`` arrays are handled alike, and a NaN
bit pattern survives a copy unchanged.

* Write (page 1, section 3(3): step 1) fills the prompt's K/V into the
  physical blocks through the block table, step 2) adds each new token's K/V
  to its block; page 3, section 03, reading (4): the worker hands the kernels
  ``slot_mapping``).  Token t goes to slot s = slot_mapping[t], i.e. block
  s // B, offset s % B.  Slots outside [0, num_blocks * B) are skipped (a
  padding token has no slot).
* Copy (page 1, section 4, step (2): the writer's shared block is duplicated
  into a fresh block before its token lands).  For every pair (src, dst) the
  whole of block dst, all heads, takes block src's contents as they were
  before the call.
"""

from __future__ import annotations

import numpy as np


def paged_kv_write(k, v, slot_mapping, k_cache, v_cache):
    """Return copies of (k_cache, v_cache) with tokens written at their slots.

    k, v: [T, num_kv_heads, head_dim]; slot_mapping: [T] integers.
    The caller keeps slots distinct (two tokens for one slot is a caller error).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    num_blocks, _, B, _ = kc.shape
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = np.nonzero((slots >= 0) & (slots < num_blocks * B))[0]
    block = slots[keep] // B
    offset = slots[keep] % B
    kc[block, :, offset, :] = np.asarray(k)[keep]
    vc[block, :, offset, :] = np.asarray(v)[keep]
    return kc, vc


def copy_blocks(k_cache, v_cache, pairs):
    """Return copies of (k_cache, v_cache) after copying each (src, dst) block."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    src_k = {int(s): np.array(k_cache[int(s)], copy=True) for s, _ in pairs}
    src_v = {int(s): np.array(v_cache[int(s)], copy=True) for s, _ in pairs}
    for s, d in pairs:
        kc[int(d)] = src_k[int(s)]
        vc[int(d)] = src_v[int(s)]
    return kc, vc
