"""CPU oracle for the paged-KV decode path.  TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously correct re-statement of what the
paged KV cache computes, written from three web pages about vLLM's
PagedAttention:

  page 1  "PagedAttention" blog post, http://www.0539edu.com/news/28468/blog.html
          (section 3 "PagedAttention原理", part (3) single request with its
          1) Prefill and 2) Decode steps; section 4 "Parallel Sampling")
  page 2  vLLM article, https://zzfmdn.com/art/... (paragraphs on the
          PagedAttention algorithm and on the vLLM system architecture)
  page 3  "Month 2 · PagedAttention", http://weishuz.com/infra-learning-path/
          tutorial/03-memory.html (section 02 OS-to-vLLM table, section 03
          source-reading anchors, section 06 misconceptions)

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it.  It shares no code with the HIP library under
``paged_kv_cache_377_amd/`` and never imports it; the product path never
imports this package.

Floating point is fp64 throughout.  bf16 tensors are carried as ``uint16`` bit
arrays and fp32 tensors as ``float32`` arrays; the oracle up-casts them
exactly (a bf16 value is the fp32 value whose top 16 bits are the bf16 bits).

Modules:
  allocator   block pool + per-sequence block tables (free list, ref counts,
              lazy allocation, fork, copy-on-write, free)
  cache_ops   slot_mapping write and block copy, on raw bit patterns
  attention   decode and causal prefill attention over K/V gathered through
              the block table
"""

from .allocator import AllocError, BlockAllocatorModel, E_INVAL, E_NOBLOCKS
from .cache_ops import copy_blocks, paged_kv_write
from .attention import paged_attention_decode, paged_attention_prefill, to_f64

__all__ = [
    "AllocError",
    "BlockAllocatorModel",
    "E_INVAL",
    "E_NOBLOCKS",
    "copy_blocks",
    "paged_kv_write",
    "paged_attention_decode",
    "paged_attention_prefill",
    "to_f64",
]
