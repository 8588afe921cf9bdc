"""Decode attention over K/V gathered through the block table, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The attention itself is ordinary softmax attention; the only difference from
the contiguous case is that key and value rows are fetched from scattered
physical blocks through the sequence's block table (page 3, section 06,
misconception 1; page 1, section 3(3), step 2): the logical blocks look
contiguous while the data is read from physical blocks; page 2, the
architecture paragraph on the "forth" query vector reading keys and values
from non-contiguous blocks).

For sequence s with n = context_lens[s] tokens and query head h:

  g       = h // G,  G = num_q_heads // num_kv_heads  (query heads h with equal
            h // G share one KV head; the pages do not mention grouped heads,
            this is the plain reading the grouped-head workloads need)
  K_t     = k_cache[block_tables[s][t // B], g, t % B, :]   for t < n
  V_t     = v_cache[block_tables[s][t // B], g, t % B, :]
  l_t     = scale * <q[s, h, :], K_t>
  out     = sum_t exp(l_t - max_u l_u) V_t / sum_t exp(l_t - max_u l_u)

and out = 0 when n = 0.  Slots at positions >= n and blocks the table does not
reach are never read, so whatever bits they hold (NaN included) cannot reach
the result.

Prefill (several new tokens per sequence; page 1, section 3(3), step 1): the
prompt's tokens are computed together and their K/V are filled into the
sequence's blocks.  Reading taken: the new tokens are the last n_new of the
sequence's n = context_lens[s] tokens (their K/V written before the
attention, as in decode), and new token j, at position p = n - n_new + j,
attends causally to every position t <= p:

  out[j] = sum_{t <= p} exp(l_t - max_{u <= p} l_u) V_t / sum_{t <= p} exp(...)

With one new token per sequence this is the decode above; with earlier
positions already cached (prefix caching, or a prompt split into chunks) the
new tokens still see the whole prefix through the table.
"""

from __future__ import annotations

import numpy as np


def to_f64(x, dtype: str):
    """Exact up-cast to fp64: 'bf16' arrays are uint16 bit patterns, 'f32'
    arrays are float32."""
    x = np.asarray(x)
    if dtype == "bf16":
        if x.dtype != np.uint16:
            raise TypeError("bf16 data must be given as uint16 bit patterns")
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        if x.dtype != np.float32:
            raise TypeError("f32 data must be float32")
        return x.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens,
                           scale: float, dtype: str, seqs=None, heads=None):
    """fp64 decode attention.  Returns out[S, Hq, D] (fp64).

    q: [S, Hq, D]; k_cache, v_cache: [NB, Hkv, B, D]; block_tables: [S, M];
    context_lens: [S].  ``seqs`` / ``heads`` restrict the work to a subset
    (the other rows of the result stay 0), for sampled checks at full size.
    """
    S, Hq, D = q.shape
    _, Hkv, B, _ = k_cache.shape
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    out = np.zeros((S, Hq, D), dtype=np.float64)
    seq_list = range(S) if seqs is None else seqs
    head_list = range(Hq) if heads is None else heads
    for s in seq_list:
        n = int(context_lens[s])
        if n == 0:
            continue
        blocks = [int(block_tables[s][t // B]) for t in range(n)]
        offsets = [t % B for t in range(n)]
        gathered = {}  # KV head -> its gathered (K, V), shared by the head's G query heads
        for h in head_list:
            g = h // G
            if g not in gathered:
                gathered[g] = (to_f64(k_cache[blocks, g, offsets, :], dtype),   # [n, D]
                               to_f64(v_cache[blocks, g, offsets, :], dtype))   # [n, D]
            K, V = gathered[g]
            qh = to_f64(q[s, h, :], dtype)                      # [D]
            logits = scale * (K @ qh)                           # [n]
            w = np.exp(logits - logits.max())
            out[s, h, :] = (w @ V) / w.sum()
    return out


def paged_attention_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                            scale: float, dtype: str, seqs=None, heads=None):
    """fp64 causal attention of new tokens over their paged context.

    q: [T, Hq, D], the new tokens of all sequences packed in sequence order;
    query_start_loc: [S + 1], sequence s owns rows query_start_loc[s] ..
    query_start_loc[s + 1] - 1.  Returns out[T, Hq, D] (fp64); rows of
    sequences outside ``seqs`` stay 0.
    """
    T, Hq, D = q.shape
    _, Hkv, B, _ = k_cache.shape
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    S = len(context_lens)
    qsl = [int(x) for x in query_start_loc]
    if len(qsl) != S + 1 or qsl[0] != 0 or qsl[-1] != T or any(b < a for a, b in zip(qsl, qsl[1:])):
        raise ValueError("query_start_loc must run from 0 to T without decreasing")
    out = np.zeros((T, Hq, D), dtype=np.float64)
    seq_list = range(S) if seqs is None else seqs
    head_list = range(Hq) if heads is None else heads
    for s in seq_list:
        n = int(context_lens[s])
        n_new = qsl[s + 1] - qsl[s]
        if n_new > n:
            raise ValueError(f"sequence {s}: {n_new} new tokens but context {n}")
        if n_new == 0:
            continue
        first = n - n_new
        blocks = [int(block_tables[s][t // B]) for t in range(n)]
        offsets = [t % B for t in range(n)]
        gathered = {}  # KV head -> its gathered (K, V), shared by the head's G query heads
        for h in head_list:
            g = h // G
            if g not in gathered:
                gathered[g] = (to_f64(k_cache[blocks, g, offsets, :], dtype),   # [n, D]
                               to_f64(v_cache[blocks, g, offsets, :], dtype))
            K, V = gathered[g]
            for j in range(n_new):
                p = first + j
                qh = to_f64(q[qsl[s] + j, h, :], dtype)
                logits = scale * (K[: p + 1] @ qh)
                w = np.exp(logits - logits.max())
                out[qsl[s] + j, h, :] = (w @ V[: p + 1]) / w.sum()
    return out
