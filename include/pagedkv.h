/*
 * pagedkv.h -- C ABI of the MI355X (gfx950) paged KV-cache decode library.
 *
 * The KV cache is cut into fixed-size physical blocks; a sequence reaches its
 * tokens through a block table that maps logical block i to a physical block
 * (PagedAttention blog, 0539edu.com, section 3(3) "PagedAttention处理单个请求").
 * This library provides the three device operations of that design and the
 * host-side block allocator that feeds them:
 *
 *   pkv_paged_kv_write          write new tokens' K/V into their slots
 *   pkv_copy_blocks             copy whole blocks (copy-on-write of shared blocks)
 *   pkv_swap_blocks             copy whole blocks between HBM and host memory
 *   pkv_paged_attention_decode  one-query-per-sequence attention through the table
 *   pkv_paged_attention_decode_append  the same with the new token's K/V written in the launch
 *   pkv_paged_attention_prefill causal attention of several new tokens per sequence
 *   pkv_alloc_* / pkv_seq_*     free list, ref counts, lazy allocation, fork, CoW
 *
 * Conventions common to every call:
 *   - Return value: PKV_OK (0) or a negative PKV_E* code.  Nothing is thrown
 *     across the ABI.  On error no kernel is launched and allocator state is
 *     unchanged; pkv_last_error() gives a message (thread-local).
 *   - Device pointers are caller-owned device memory (the library never
 *     allocates or frees device memory).  Host pointers are caller-owned host
 *     memory.  `stream` is a hipStream_t passed as void* (NULL = null stream);
 *     every device call is asynchronous on it and does no device->host sync.
 *   - Cache layout (both K and V): [num_blocks, num_kv_heads, block_size,
 *     head_dim], contiguous, element type `dtype`.  One (block, head) pair is
 *     one contiguous run of block_size * head_dim elements.
 *   - Compiled instances: dtype in {PKV_F32, PKV_BF16}, head_dim in {64, 128},
 *     block_size in {8, 16, 32}, query heads per KV head in {1, 2, 4, 8}.
 *     Other shapes return PKV_EUNSUPPORTED.
 *   - The allocator is not thread-safe: one scheduler thread owns a handle.
 *   - Debugging: with PKV_VALIDATE set to anything but "0" in the environment
 *     (read on every call), each device call first copies its index arrays
 *     (slots, copy pairs, tables, lengths, row starts) to the host,
 *     synchronously on its stream, and checks them by the rules of the
 *     pkv_validate_* calls below; a violation returns PKV_ERANGE and nothing
 *     is launched.  This waits for the stream: not for timing or graph
 *     capture.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,       /* bad shape, dtype, id or argument                  */
  PKV_ENOBLOCKS = -2,    /* the pool cannot supply the blocks a call needs     */
  PKV_ERANGE = -3,       /* a validate call found an out-of-contract value     */
  PKV_EHIP = -4,         /* a HIP launch or runtime call failed                */
  PKV_EUNSUPPORTED = -5  /* (dtype, head_dim, block_size, group) not compiled  */
};

enum { PKV_F32 = 0, PKV_BF16 = 1 };

typedef struct {
  int32_t num_blocks;    /* physical blocks in the pool                       */
  int32_t num_kv_heads;
  int32_t block_size;    /* tokens per block                                  */
  int32_t head_dim;
  int32_t dtype;         /* PKV_F32 or PKV_BF16                               */
} pkv_cache_desc;

/* ------------------------------------------------------------------------ */
/* Device operations                                                         */
/* ------------------------------------------------------------------------ */

/*
 * Write the K/V of `num_tokens` new tokens into the cache through their slots
 * (blog section 3(3): prefill fills the prompt's K/V into the physical blocks,
 * each decode step adds the new token's K/V to its block; weishuz.com Month 2
 * section 03, reading (4): the worker hands the kernels `slot_mapping`).
 *
 *   k, v          device, [num_tokens, num_kv_heads, head_dim], dtype c->dtype
 *   slot_mapping  device, [num_tokens] int64; token t goes to block
 *                 slot / block_size, offset slot % block_size, every head.
 *                 Slots outside [0, num_blocks * block_size) are skipped.
 *                 Two tokens naming one slot is a caller error (the result
 *                 is then unspecified; pkv_validate_write reports it).
 *   k_cache, v_cache  device, cache layout, updated in place.
 * num_tokens == 0 launches nothing.  Errors: PKV_EINVAL (null pointer,
 * negative count, bad desc), PKV_EUNSUPPORTED, PKV_EHIP.
 */
int pkv_paged_kv_write(const void* k, const void* v, const int64_t* slot_mapping,
                       int32_t num_tokens, void* k_cache, void* v_cache,
                       const pkv_cache_desc* c, void* stream);

/*
 * Copy whole blocks, all heads, K and V: block dst takes block src's contents
 * (blog section 4 "Parallel Sampling", step (2): the sample that writes into
 * a shared block first gets its own copy of it).
 *
 *   src_dst_pairs  device, [num_pairs][2] int32 {src, dst}.  Contract: every
 *                  id in [0, num_blocks), dsts distinct, no dst is also a src
 *                  (so every read sees pre-call contents).  A src may repeat.
 * Pairs outside [0, num_blocks) are skipped by the kernel; the other contract
 * violations give unspecified contents (pkv_validate_copy reports them).
 * num_pairs == 0 launches nothing.  Errors: PKV_EINVAL, PKV_EHIP.
 */
int pkv_copy_blocks(void* k_cache, void* v_cache, const pkv_cache_desc* c,
                    const int32_t* src_dst_pairs, int32_t num_pairs, void* stream);

/* Size of the per-device array pkv_paged_attention_decode_noalloc works in. */
#define PKV_DECODE_NOALLOC_MAX_BYTES ((size_t)32 << 20)

/* partition_size value: let the library split the work (see below). */
enum { PKV_PARTITION_AUTO = -1 };

/*
 * Bytes of device workspace pkv_paged_attention_decode needs for these sizes
 * and this partition_size, on the current HIP device (0 when the call needs
 * none, and 0 with pkv_last_error() set on invalid arguments).  With
 * PKV_PARTITION_AUTO the figure depends on the device's compute-unit count,
 * so size the workspace on the device that runs the decode.
 */
size_t pkv_decode_workspace_bytes(const pkv_cache_desc* c, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t max_context_len,
                                  int32_t partition_size);

/*
 * The most sequences one balanced-split decode takes on the current HIP
 * device (-1 with pkv_last_error() set if the device cannot be queried).
 * Every workgroup of that split keeps each sequence's context length and
 * tile prefix sum in LDS, 8 bytes per sequence, within the LDS one of its
 * workgroups may use (one workgroup per compute unit): 20475 sequences on
 * MI355X's 160 KiB.  Larger batches run in split-context partitions of 512
 * tokens.
 */
int32_t pkv_decode_balanced_max_seqs(void);

/*
 * Decode attention: one query token per sequence against that sequence's
 * cached K/V, read through its block table (blog section 3(3), step 2:
 * attention is computed over the logically contiguous tokens while the data
 * comes from physical blocks; weishuz.com Month 2, section 06: the kernel is
 * ordinary attention whose only difference is gathering K and V from
 * non-contiguous addresses; section 02: the block table lives in GPU memory
 * and the lookup happens inside the kernel).
 *
 * For sequence s with n = context_lens[s] and query head h, G = num_q_heads /
 * c->num_kv_heads, g = h / G:
 *   K_t = k_cache[block_tables[s*max_blocks_per_seq + t/B], g, t%B, :], t < n
 *   out[s,h,:] = sum_t softmax_t(scale * <q[s,h,:], K_t>) * V_t   (0 if n == 0)
 * computed in fp32 from dtype inputs and rounded to dtype (bf16:
 * round-to-nearest-even).
 *
 *   out           device, [num_seqs, num_q_heads, head_dim], dtype
 *   q             device, [num_seqs, num_q_heads, head_dim], dtype
 *   block_tables  device, [num_seqs, max_blocks_per_seq] int32; the first
 *                 ceil(context_lens[s] / block_size) entries of row s are used
 *                 and each must be in [0, num_blocks) (an entry outside the
 *                 pool is never dereferenced; the result is then unspecified);
 *                 later entries of the row may be read but are never used
 *   context_lens  device, [num_seqs] int32, each in [0, max_context_len]; it
 *                 counts the token just written by pkv_paged_kv_write
 *   max_context_len  host int, bound on context_lens (sizes the launch)
 *   partition_size   how the work is split:
 *                 PKV_PARTITION_AUTO: bf16 caches with num_seqs <=
 *                   pkv_decode_balanced_max_seqs() use a balanced split: every worker wave of the GPU reads an
 *                   equal share of all sequences' 16-token tiles (ragged
 *                   context lengths cannot unbalance it), and the sequences
 *                   whose tiles several workers share are combined by a second
 *                   kernel; otherwise as partition_size 512;
 *                 a positive multiple of block_size: split-context partitions
 *                   of that many tokens, one workgroup each, then a combine
 *                   kernel when a sequence spans several;
 *                 0: no split (one workgroup per sequence and KV head).
 *   workspace     device, >= pkv_decode_workspace_bytes(...) bytes (may be
 *                 NULL when that is 0), 16-byte aligned; contents need no
 *                 initialisation and are scratch between calls
 * Slots at positions >= n and blocks the table does not reach are never
 * used (any bits, NaN included, leave the result unchanged).  The result does
 * not depend on physical block ids and is the same on every run (no atomics;
 * every combine runs in a fixed order).  Calls that share one workspace must
 * be ordered (one stream).
 * Errors: PKV_EINVAL (null pointer, bad sizes, workspace too small, partition
 * size not allowed), PKV_EUNSUPPORTED, PKV_EHIP.
 */
int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                               const void* v_cache, const pkv_cache_desc* c,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t max_context_len, float scale,
                               int32_t partition_size, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * pkv_paged_attention_decode without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The workspace is a
 * library-owned device array of PKV_DECODE_NOALLOC_MAX_BYTES bytes
 * (32 MiB), one per device, held until the process ends; its address is
 * looked up on the first call made on a device and the call allocates
 * nothing.  Arguments, results and errors as pkv_paged_attention_decode,
 * plus PKV_EINVAL when pkv_decode_workspace_bytes(...) for these sizes
 * exceeds the array (nothing is launched then): 17 MiB is the most any of
 * the decode workloads here needs (256 sequences, 8 KV heads, G = 8).
 * Nothing in the array needs to start at zero: every call writes what it
 * reads.  All calls on one device share its array, so calls on one device
 * that may overlap (different streams, or host threads without ordering)
 * race and give unspecified results; calls ordered on one stream do not.
 */
int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const pkv_cache_desc* c,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t max_context_len,
                                       float scale, int32_t partition_size, void* stream);

/*
 * Append + decode in one launch: for each sequence s with n = context_lens[s]
 * >= 1, the new token's K/V rows k_new[s], v_new[s] ([num_seqs, Hkv, D],
 * dtype) are written to the slot of position n - 1 (block
 * block_tables[s][(n - 1) / B], offset (n - 1) % B), and the decode of
 * pkv_paged_attention_decode runs over positions 0..n-1 with the appended row
 * read from k_new / v_new.  Same results, bit for bit, as pkv_paged_kv_write of
 * those rows followed by pkv_paged_attention_decode, with one launch fewer.
 * The slot of position n - 1 must not be shared with another sequence (the
 * allocator's copy-on-write guarantees this; run pkv_copy_blocks first).
 * Sequences with n = 0 append nothing.  Runs the balanced split only: bf16
 * caches and num_seqs <= pkv_decode_balanced_max_seqs() (PKV_EUNSUPPORTED
 * otherwise).  Workspace as for
 * pkv_decode_workspace_bytes(..., PKV_PARTITION_AUTO).
 * Errors: as pkv_paged_attention_decode.
 */
int pkv_paged_attention_decode_append(void* out, const void* q, const void* k_new,
                                      const void* v_new, void* k_cache, void* v_cache,
                                      const pkv_cache_desc* c, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_q_heads,
                                      int32_t max_context_len, float scale, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * Causal attention of several new tokens per sequence over the sequence's
 * paged context (blog section 3(3), step 1: a prompt's tokens are processed
 * together and their K/V are filled into the sequence's blocks; the K/V of
 * the new tokens are written with pkv_paged_kv_write before this call).
 * Sequence s owns query rows query_start_loc[s] .. query_start_loc[s+1] - 1:
 * its n_new new tokens, the last n_new of its n = context_lens[s] tokens.  New
 * token j (position p = n - n_new + j) and query head h (KV head h / G) give
 *   out[row, h, :] = sum_{t <= p} softmax_t(scale * <q[row, h, :], K_t>) V_t
 * with K_t, V_t read through the table as in decode.  One new token per
 * sequence is the decode; tokens before the new ones may come from the prefix
 * cache or from earlier chunks of the same prompt.  Computed on MFMA with
 * fp32 accumulation; each softmax weight enters the V product as two bf16
 * parts (bf16(p) and bf16 of the remainder, nearest even), and the output is
 * rounded to bf16 (nearest even).
 *
 *   out, q           device, [num_tokens, num_q_heads, head_dim] bf16
 *   block_tables     device, [num_seqs, max_blocks_per_seq] int32, as in decode
 *   context_lens     device, [num_seqs] int32, each in [n_new, max_context_len]
 *   query_start_loc  device, [num_seqs + 1] int32, non-decreasing, from 0 to
 *                    at most num_tokens
 *   max_new_tokens   host int, >= every n_new (sizes the launch)
 *   max_context_len  host int, >= every context_lens[s]
 *   scale            finite and > 0 (PKV_EINVAL otherwise)
 * Positions after a row's own never affect it; slots at positions >= n and
 * blocks the table does not reach are never used.  Bad device-side contents
 * (n_new > n, table entries outside the pool) never lead to an access
 * outside the arrays; the result is then unspecified.  Only bf16 caches,
 * head_dim in {64, 128}, block_size in {8, 16, 32} and query heads per KV
 * head in {1, 2, 4, 8, 16} are built; other shapes return PKV_EUNSUPPORTED.
 * Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EHIP.
 */
int pkv_paged_attention_prefill(void* out, const void* q, const void* k_cache,
                                const void* v_cache, const pkv_cache_desc* c,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, const int32_t* query_start_loc,
                                int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                int32_t max_new_tokens, int32_t max_context_len, float scale,
                                void* stream);

/* ------------------------------------------------------------------------ */
/* Host-side contract checks (synchronous, for debugging; no GPU needed).    */
/* Each takes HOST copies of the index arrays and returns PKV_OK, PKV_ERANGE */
/* (message names the first offending index) or PKV_EINVAL (bad arguments). */
/* ------------------------------------------------------------------------ */

/* in-range slots are pairwise distinct */
int pkv_validate_write(const int64_t* slot_mapping, int32_t num_tokens,
                       const pkv_cache_desc* c);
/* ids in range, dsts distinct, no dst is a src */
int pkv_validate_copy(const int32_t* src_dst_pairs, int32_t num_pairs,
                      const pkv_cache_desc* c);
/* query_start_loc runs from 0 to <= num_tokens without decreasing, every
 * n_new <= max_new_tokens and <= its context length, plus the decode checks */
int pkv_validate_prefill(const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, const int32_t* query_start_loc,
                         int32_t num_seqs, int32_t num_tokens, int32_t max_new_tokens,
                         int32_t max_context_len, const pkv_cache_desc* c);
/* 0 <= ctx <= max_context_len, ceil(ctx/B) <= width, read entries in range */
int pkv_validate_decode(const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t num_seqs,
                        int32_t max_context_len, const pkv_cache_desc* c);

/* ------------------------------------------------------------------------ */
/* Host block allocator                                                      */
/* ------------------------------------------------------------------------ */
/*
 * The pool keeps a FIFO free list and a reference count per physical block
 * (weishuz.com Month 2, section 03 reading (2): the block pool's free list;
 * section 04: ref_cnt).  Blocks are taken from the head of the free list and
 * returned to its tail.  A new block is taken only when a token crosses into
 * a block the sequence has not mapped yet (section 02, row "page fault": lazy
 * allocation).  A token appended into a shared, partially filled last block
 * first copies that block (blog section 4, step (2)).  Sequence ids are
 * arbitrary int64 values chosen by the caller.
 */

typedef struct pkv_alloc pkv_alloc;

typedef struct {
  int32_t num_blocks;
  int32_t num_free;
  int32_t block_size;
  int32_t num_seqs;
  int64_t capacity_tokens;   /* num_blocks * block_size                        */
  int64_t allocated_slots;   /* (num_blocks - num_free) * block_size            */
  int64_t filled_slots;      /* filled slots of blocks in use, each block once  */
  int64_t logical_tokens;    /* sum of sequence lengths (shared tokens repeat)  */
  double utilization;        /* filled_slots / allocated_slots (0 if none)      */
} pkv_stats;

/* Largest block size the allocator accepts (the kernels are built for 8, 16
 * and 32). */
#define PKV_MAX_BLOCK_SIZE 65536

/*
 * New pool of `num_blocks` blocks of `block_size` tokens.  free_order: host
 * [num_blocks] permutation of 0..num_blocks-1 giving the free list from head
 * to tail, or NULL for ascending ids.  Returns NULL on bad arguments or
 * out of host memory (pkv_last_error() says which).  The handle is owned by
 * the library: release it with pkv_alloc_destroy.
 */
pkv_alloc* pkv_alloc_create(int32_t num_blocks, int32_t block_size,
                            const int32_t* free_order);
void pkv_alloc_destroy(pkv_alloc* a);

/*
 * Admit sequence `seq` holding `num_tokens` tokens (its prompt): takes
 * ceil(num_tokens / block_size) blocks (blog section 3(3), step 1)).  slots_out:
 * host [num_tokens] or NULL; receives the slot of every position.
 * Errors: PKV_EINVAL (seq exists, num_tokens < 0), PKV_ENOBLOCKS.
 */
int pkv_seq_add(pkv_alloc* a, int64_t seq, int32_t num_tokens, int64_t* slots_out);

/* `child` starts as a copy of `parent`: same table and length, every block
 * gains a reference (blog section 4, step (1)).  Errors: PKV_EINVAL. */
int pkv_seq_fork(pkv_alloc* a, int64_t parent, int64_t child);

/*
 * Reserve the slot of one new token of `seq`.  cow_out (host [2], may be
 * NULL) receives {src, dst} when the shared last block had to be copied
 * first (the caller runs pkv_copy_blocks before writing the token), else
 * {-1, -1}.  Errors: PKV_EINVAL, PKV_ENOBLOCKS.
 */
int pkv_seq_append(pkv_alloc* a, int64_t seq, int64_t* slot_out, int32_t cow_out[2]);

/*
 * One decode step: append one token to each of seqs[0..n-1], in array order.
 * All-or-nothing: the blocks the whole step needs are counted first; if the
 * pool has fewer, nothing changes and PKV_ENOBLOCKS is returned with the
 * message "failed to allocate K blocks: F free of N total" (weishuz.com Month 2,
 * section 07: such a message should state the pool size).
 *   slots_out      host [n] int64
 *   cow_pairs_out  host [n][2] int32 (at most one copy per sequence)
 *   num_cow_out    host, number of pairs written
 * Errors: PKV_EINVAL (unknown or repeated id, n < 0), PKV_ENOBLOCKS.
 */
int pkv_step_append(pkv_alloc* a, const int64_t* seqs, int32_t n, int64_t* slots_out,
                    int32_t* cow_pairs_out, int32_t* num_cow_out);

/* Release a sequence: its blocks are visited from the last to the first, and
 * each one whose count reaches 0 goes to the free-list tail.  Errors: PKV_EINVAL. */
int pkv_seq_free(pkv_alloc* a, int64_t seq);

/* Length and block count of one sequence.  Errors: PKV_EINVAL. */
int pkv_seq_info(const pkv_alloc* a, int64_t seq, int32_t* len_out, int32_t* num_blocks_out);

/*
 * Block tables for seqs[0..n-1]: tables_out host [n][width] int32 (entries
 * past a sequence's last block are 0 and are never read by the decode),
 * ctx_lens_out host [n] int32.  Errors: PKV_EINVAL (unknown id, a sequence
 * holding more than `width` blocks).
 */
int pkv_build_tables(const pkv_alloc* a, const int64_t* seqs, int32_t n,
                     int32_t* tables_out, int32_t width, int32_t* ctx_lens_out);

/* Pool counters (weishuz.com Month 2, section 05: KV cache size and
 * utilisation; section 07: free-block count). */
int pkv_alloc_stats(const pkv_alloc* a, pkv_stats* out);

/* Copy out the free list (head to tail) and the reference counts:
 * free_fifo_out host [num_blocks] (first *num_free_out entries written),
 * ref_cnt_out host [num_blocks]. */
int pkv_alloc_export(const pkv_alloc* a, int32_t* free_fifo_out, int32_t* num_free_out,
                     int32_t* ref_cnt_out);

/*
 * The pages say nothing about saving an allocator; these calls exist so that
 * a process can persist, move or replay the manager's state (and a test can
 * compare it word for word with a reference model).
 *
 * Checkpoint and restore of the whole allocator state: free-list order,
 * reference counts, every live sequence (id, length, block table, and the
 * token ids and chain hash it enters prefix-cache blocks with), the prefix
 * cache (entries and hit/query/eviction counters) and the host pool (free
 * list and counts).  A handle restored from a saved state answers every later
 * call as the saved one would.  The state is a flat array of int64 words,
 * little-endian as the host writes them:
 *   magic "PKVSTATE", version 1, num_blocks, block_size, prefix caching on,
 *   host blocks, free blocks F, live sequences S, cached blocks C, hits,
 *   queries, evictions, free host blocks FH;
 *   the free list head to tail (F words); the reference counts (num_blocks);
 *   per sequence, ids ascending: id, length, block count n, flags (1: token
 *   ids tracked, 2: swapped out), chain hash, the n table entries, then
 *   block_size token ids when tracked;
 *   per cached block, ids ascending: block, key, parent key, its block_size
 *   token ids; the host free list head to tail (FH); the host counts.
 *
 * pkv_alloc_save_bytes: bytes the current state needs (0 and an error on a
 *   NULL handle).
 * pkv_alloc_save: writes the state to buf (host, >= that many bytes) and the
 *   byte count to *written (may be NULL).  Errors: PKV_EINVAL.
 * pkv_alloc_restore: a new handle (owned by the caller, released with
 *   pkv_alloc_destroy) holding a saved state; NULL with pkv_last_error() set
 *   when the words are not a consistent state (bad magic or sizes, ids out of
 *   range, counts that disagree with the tables and free lists, trailing
 *   words).
 * pkv_alloc_seq_ids: the live sequence ids, ascending, into ids_out (host,
 *   max_ids entries); *num_out receives their count.  Errors: PKV_EINVAL
 *   (including max_ids below the count).
 */
size_t pkv_alloc_save_bytes(const pkv_alloc* a);
int pkv_alloc_save(const pkv_alloc* a, void* buf, size_t bytes, size_t* written);
pkv_alloc* pkv_alloc_restore(const void* buf, size_t bytes);
int pkv_alloc_seq_ids(const pkv_alloc* a, int64_t* ids_out, int32_t max_ids, int32_t* num_out);

/*
 * Prefix caching (weishuz.com Month 2, section 04: a computed prompt's K/V
 * stay in device memory and a later prompt with the same leading tokens maps
 * the same blocks instead of computing them again; section 03 reading (2): a
 * map from block hash to block beside the free list; section 07: hit-rate
 * metric).
 *
 * Keys: full blocks only.  The key of logical block i is the chain hash
 * h_i = H(h_{i-1}, ids of its B tokens), so it covers the whole prefix; a hit
 * also compares the block's ids and h_{i-1}.  A full block is entered once the
 * tokens that fill it have slots: prompt blocks by pkv_seq_add_tokens, later
 * blocks by appends that carry token ids; under an existing key the first
 * block entered stays.  A block whose count drops to 0 stays cached in the
 * free list (release order); a hit takes it back out; the free list hands out
 * its head and that block's entry is then evicted (least recently released
 * first; a referenced block is never evicted).
 */
typedef struct {
  int32_t enabled;
  int32_t cached_blocks;     /* blocks currently in the map                     */
  int64_t queries;           /* full prompt blocks looked up                    */
  int64_t hits;              /* of those, found in the cache                    */
  int64_t evictions;         /* cached blocks handed out again                  */
  double hit_rate;           /* hits / queries (0 if none)                      */
} pkv_prefix_stats;

/* Turn prefix caching on.  Only before the first sequence is added
 * (PKV_EINVAL otherwise); it stays on for the handle's life. */
int pkv_prefix_cache_enable(pkv_alloc* a);

/*
 * Admit `seq` with its prompt's token ids tokens[0..num_tokens-1] (host).
 * With prefix caching, the prompt's leading full blocks found in the cache
 * are mapped (the walk stops at the first miss) and *num_cached_out (may be
 * NULL) receives the number of leading positions whose K/V the pool already
 * holds (a multiple of block_size): the caller writes K/V only for positions
 * from there on.  The hits are taken back first, then fresh blocks from the
 * free-list head, then the missed full blocks are entered.  slots_out: host
 * [num_tokens] or NULL.  All-or-nothing; PKV_ENOBLOCKS counts the blocks
 * this call takes off the free list (fresh ones and hits with count 0).
 * Without prefix caching it behaves as pkv_seq_add.
 */
int pkv_seq_add_tokens(pkv_alloc* a, int64_t seq, const int32_t* tokens, int32_t num_tokens,
                       int64_t* slots_out, int32_t* num_cached_out);

/* pkv_seq_append / pkv_step_append with the new tokens' ids (host; tokens[i]
 * belongs to seqs[i]).  A block such a token fills is entered in the cache.
 * The plain calls append tokens of unknown id: the sequence then stops
 * entering blocks. */
int pkv_seq_append_token(pkv_alloc* a, int64_t seq, int32_t token, int64_t* slot_out,
                         int32_t cow_out[2]);
int pkv_step_append_tokens(pkv_alloc* a, const int64_t* seqs, const int32_t* tokens, int32_t n,
                           int64_t* slots_out, int32_t* cow_pairs_out, int32_t* num_cow_out);

/* Read-only lookup (the manager's get_cached_blocks(), section 03 reading
 * (1)): the cached blocks a prompt of these ids would map.  blocks_out: host
 * [num_tokens / block_size]; *num_blocks_out receives the count (0 when
 * prefix caching is off).  Changes no counter. */
int pkv_prefix_cache_lookup(const pkv_alloc* a, const int32_t* tokens, int32_t num_tokens,
                            int32_t* blocks_out, int32_t* num_blocks_out);

int pkv_prefix_cache_stats(const pkv_alloc* a, pkv_prefix_stats* out);

/*
 * Swapping (weishuz.com Month 2, section 02, row "swap to disk": blocks of a
 * preempted request move to host memory and come back later).  The handle
 * gets a second pool of host blocks; a group of sequences moves between the
 * pools as a whole.  Every distinct block the group maps (first appearance
 * in array order, then table order) gets a block from the target pool's
 * free-list head and keeps its reference count; pairs_out receives the
 * (source id, target id) pairs in that order, for pkv_swap_blocks; the
 * source blocks are then released last pair first.  The pairs must be copied
 * before the released blocks are reused (the next call that allocates).
 * All-or-nothing.  Errors: PKV_EINVAL (no host pool, a sequence unknown,
 * repeated or in the other pool, a block shared with a sequence outside the
 * group, max_pairs below the group's table entries), PKV_ENOBLOCKS (target
 * pool short; the message names the target pool's size).  A swapped-out
 * sequence cannot append, fork or be tabled; pkv_seq_free releases its host
 * blocks.
 */
int pkv_alloc_set_host_pool(pkv_alloc* a, int32_t num_host_blocks, const int32_t* free_order);
int pkv_seq_swap_out(pkv_alloc* a, const int64_t* seqs, int32_t n, int32_t* pairs_out,
                     int32_t max_pairs, int32_t* num_pairs_out);
int pkv_seq_swap_in(pkv_alloc* a, const int64_t* seqs, int32_t n, int32_t* pairs_out,
                    int32_t max_pairs, int32_t* num_pairs_out);
int pkv_seq_swapped(const pkv_alloc* a, int64_t seq, int32_t* swapped_out);
/* host pool's free list (head to tail) and reference counts, as pkv_alloc_export */
int pkv_host_pool_export(const pkv_alloc* a, int32_t* free_fifo_out, int32_t* num_free_out,
                         int32_t* ref_cnt_out);

/*
 * Copy whole blocks between two pools of the same block shape (c gives
 * num_kv_heads, block_size, head_dim, dtype; c->num_blocks is ignored):
 * for each i, K and V block pairs[i][1] of the destination pool take the
 * contents of block pairs[i][0] of the source pool.  Either pool may be host
 * memory the GPU can address (pinned, e.g. hipHostMalloc); this is how
 * swapped blocks move between HBM and host memory, and the copy is then
 * bound by the host link.
 *   dst_k, dst_v     [dst_num_blocks, Hkv, B, D]
 *   src_k, src_v     [src_num_blocks, Hkv, B, D]
 *   pairs            device or pinned host, [num_pairs][2] int32 (src, dst)
 * Ids outside their pool are skipped.  Destination blocks must be distinct
 * and the pools must not overlap.  Errors: PKV_EINVAL, PKV_EHIP.
 */
int pkv_swap_blocks(void* dst_k, void* dst_v, int32_t dst_num_blocks, const void* src_k,
                    const void* src_v, int32_t src_num_blocks, const pkv_cache_desc* c,
                    const int32_t* pairs, int32_t num_pairs, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
