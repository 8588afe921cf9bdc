/*
 * pagedkv_measure.h -- measurement calls of libpagedkv.so (not part of the
 * attention path).
 *
 * The decode is bound by the gather of K and V rows from scattered physical
 * blocks (weishuz.com Month 2, section 06, misconception 1; PagedAttention
 * blog, 0539edu.com, section 3(3)).  pkv_measure_gather times the memory
 * system on that access pattern alone: it reads a list of (block, KV head)
 * runs of both pools with no arithmetic, so a benchmark can put the decode's
 * time beside the time the same bytes need in the same order.
 */
#ifndef PAGEDKV_MEASURE_H
#define PAGEDKV_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read runs[0 .. num_runs-1] of both pools.  Run r is (block r / Hkv, KV head
 * r % Hkv): the block_size x head_dim elements of K and of V that sit
 * contiguously in the cache layout of pagedkv.h (4 KiB each at block 16,
 * head_dim 128, bf16; built for runs of 1, 2, 4 and 8 KiB).  Wave w of the
 * num_workers waves reads runs [w n / W, (w + 1) n / W) in order, the share
 * rule of the balanced decode, keeping runs_in_flight (1 to 3) runs' loads in
 * flight; sink[w] receives the XOR of the words it read.
 *
 *   k_pool, v_pool  device, [c->num_blocks, Hkv, B, D], 16-byte aligned
 *   runs            device, [num_runs] int32; ids outside
 *                   [0, num_blocks * Hkv) read run 0
 *   sink            device, [num_workers] uint32, written
 * At most 4096 runs per wave.  Asynchronous on `stream`.  Errors: PKV_EINVAL,
 * PKV_EUNSUPPORTED (another run size), PKV_EHIP.
 */
int pkv_measure_gather(const void* k_pool, const void* v_pool, const pkv_cache_desc* c,
                       const int32_t* runs, int64_t num_runs, int32_t num_workers,
                       int32_t runs_in_flight, uint32_t* sink, void* stream);

/*
 * Time one kernel of a decode call.  A decode call launches two kernels (the
 * partition or balanced-split kernel, then the combine or reduce kernel when
 * the split needs one), so events placed around the call time both.  After
 * this call, the next decode call made from the same thread (any of
 * pkv_paged_attention_decode, pkv_paged_attention_decode_append,
 * pkv_paged_attention_decode_noalloc) launches its first kernel with
 * hipExtLaunchKernel and the pair as that launch's start and stop events, so
 * they hold the kernel's own start and end; that call clears the pair
 * whatever it returns, and a call that launches nothing (an error, no
 * sequences) records neither.  The calls after it record nothing until the
 * next pkv_decode_mark_next_call.
 *
 *   before, after   hipEvent_t handles created by the caller (both, or both
 *                   NULL to clear a pending pair)
 * Not for use while the stream is being captured into a graph.  Errors:
 * PKV_EINVAL (exactly one NULL); a failed launch returns PKV_EHIP from the
 * decode call.
 */
int pkv_decode_mark_next_call(void* before, void* after);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_MEASURE_H */
