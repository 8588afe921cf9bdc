"""MI355X-native paged KV cache: decode and causal prefill attention,
slot_mapping write, block copy and host block allocator (with prefix
caching), behind the C ABI of include/pagedkv.h.

The Python layer is a thin ctypes binding over ``libpagedkv.so`` (built
in-tree for gfx950 by ``python -m paged_kv_cache_377_amd.build``); it loads
the library on first use and raises if it is missing.
"""

from ._lib import (  # noqa: F401
    PKV_BF16,
    PKV_EHIP,
    PKV_EINVAL,
    PKV_ENOBLOCKS,
    PKV_ERANGE,
    PKV_EUNSUPPORTED,
    PKV_F32,
    PKV_PARTITION_AUTO,
    PKV_OK,
    BlockAllocator,
    CacheDesc,
    PagedKVError,
    cache_desc,
    copy_blocks,
    decode_balanced_max_seqs,
    decode_mark_next_call,
    decode_workspace_bytes,
    header_functions,
    lib,
    measure_gather,
    paged_attention_decode,
    paged_attention_decode_append,
    paged_attention_decode_noalloc,
    decode_noalloc_max_bytes,
    paged_attention_prefill,
    paged_kv_write,
    swap_blocks,
    validate_copy,
    validate_decode,
    validate_prefill,
    validate_write,
)
