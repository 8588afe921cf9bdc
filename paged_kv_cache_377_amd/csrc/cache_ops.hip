// slot_mapping write and block copy for gfx950.
//
// Both kernels move bits, never values: every (token, head) row and every
// (block, head) run is copied in 16-byte pieces (global_load/store_dwordx4),
// so one wave moves a contiguous 1 KiB and the element type does not matter.
//
//  * Write (PagedAttention blog, 0539edu.com, section 3(3): the prompt's K/V
//    are filled into the physical blocks, and each decode step adds the new
//    token's K/V to its block; weishuz.com Month 2, section 03, reading (4):
//    the worker passes `slot_mapping` to the kernels).  Token t, head h goes
//    to block slot/B, offset slot%B.  Slots outside the pool are skipped.
//  * Copy (blog section 4, step (2): a sample writing into a shared block
//    first gets its own copy of it).  Block dst, all heads, K and V, takes
//    block src's contents.
#include <hip/hip_runtime.h>

#include <stdlib.h>

#include <stdint.h>

#include "pkv_internal.h"

namespace {

constexpr int kThreads = 256;

// One thread per 16-byte piece of the [T, Hkv, D] input.  `row_chunks` is
// D * elem_bytes / 16 and `total_chunks` = T * Hkv * row_chunks < 2^31 (the
// host checks), so the index arithmetic stays in 32 bits.
__global__ __launch_bounds__(kThreads) void kv_write_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v,
    const int64_t* __restrict__ slot_mapping, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, uint32_t num_kv_heads, uint32_t block_size,
    uint32_t row_chunks, uint32_t total_chunks, int64_t num_slots) {
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= total_chunks) return;
  const uint32_t row = i / row_chunks;
  const uint32_t c = i - row * row_chunks;
  const uint32_t t = row / num_kv_heads;
  const uint32_t h = row - t * num_kv_heads;
  const int64_t slot = slot_mapping[t];
  uint4 kv = k[i];
  uint4 vv = v[i];
  // The row loads do not depend on the slot: the empty asm needs their values
  // before the slot test, so all three loads are in flight together instead
  // of the row loads waiting for the slot.
  asm volatile("" : "+v"(kv.x), "+v"(kv.y), "+v"(kv.z), "+v"(kv.w), "+v"(vv.x), "+v"(vv.y),
               "+v"(vv.z), "+v"(vv.w));
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * row_chunks + c;
  k_cache[dst] = kv;
  v_cache[dst] = vv;
}

// Grid: num_pairs * groups_per_block workgroups; each thread copies one
// 16-byte piece of one block's K run and the same piece of its V run.  One
// piece per thread, held in registers: with several pieces per thread in a
// private array the compiler moved the array to LDS and scratch, and the copy
// ran about three times slower.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
    const int32_t* __restrict__ pairs, int32_t block_chunks, int32_t groups_per_block,
    int32_t num_blocks) {
  const int32_t pair = blockIdx.x / groups_per_block;
  const int32_t grp = blockIdx.x - pair * groups_per_block;
  const int32_t c = grp * kThreads + threadIdx.x;
  const int32_t src = pairs[2 * pair];
  const int32_t dst = pairs[2 * pair + 1];
  if (c >= block_chunks || src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const uint4 kr = k_cache[(int64_t)src * block_chunks + c];
  const uint4 vr = v_cache[(int64_t)src * block_chunks + c];
  k_cache[(int64_t)dst * block_chunks + c] = kr;
  v_cache[(int64_t)dst * block_chunks + c] = vr;
}

// Swap copy: like copy_blocks, but source and destination are two pools
// (either may be pinned host memory); one 16-byte piece of K and of V per
// thread.
__global__ __launch_bounds__(kThreads) void swap_blocks_kernel(
    uint4* __restrict__ dst_k, uint4* __restrict__ dst_v, int32_t dst_num_blocks,
    const uint4* __restrict__ src_k, const uint4* __restrict__ src_v, int32_t src_num_blocks,
    const int32_t* __restrict__ pairs, int32_t block_chunks, int32_t groups_per_block) {
  const int32_t pair = blockIdx.x / groups_per_block;
  const int32_t grp = blockIdx.x - pair * groups_per_block;
  const int32_t c = grp * kThreads + threadIdx.x;
  const int32_t src = pairs[2 * pair];
  const int32_t dst = pairs[2 * pair + 1];
  if (c >= block_chunks || src < 0 || src >= src_num_blocks || dst < 0 || dst >= dst_num_blocks)
    return;
  const uint4 kr = src_k[(int64_t)src * block_chunks + c];
  const uint4 vr = src_v[(int64_t)src * block_chunks + c];
  dst_k[(int64_t)dst * block_chunks + c] = kr;
  dst_v[(int64_t)dst * block_chunks + c] = vr;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(int32_t dtype) { return dtype == PKV_BF16 ? 2 : 4; }

}  // namespace

extern "C" int pkv__copy_to_host(void* dst, const void* src, size_t bytes, void* stream) {
  hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDefault, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return pkv__fail(PKV_EHIP, "validation copy: %s", hipGetErrorString(e));
  return PKV_OK;
}

namespace {

// PKV_VALIDATE checks of the index arrays of a write, a copy and a swap.
int validate_write_device(const int64_t* slots, int32_t n, const pkv_cache_desc* c, void* stream) {
  int64_t* h = (int64_t*)malloc((size_t)n * sizeof(int64_t));
  if (!h) return pkv__fail(PKV_EINVAL, "out of host memory");
  int rc = pkv__copy_to_host(h, slots, (size_t)n * sizeof(int64_t), stream);
  if (!rc) rc = pkv_validate_write(h, n, c);
  free(h);
  return rc;
}

int validate_pairs_device(const int32_t* pairs, int32_t n, int32_t src_blocks, int32_t dst_blocks,
                          const pkv_cache_desc* c, bool same_pool, void* stream) {
  int32_t* h = (int32_t*)malloc((size_t)n * 2 * sizeof(int32_t));
  if (!h) return pkv__fail(PKV_EINVAL, "out of host memory");
  int rc = pkv__copy_to_host(h, pairs, (size_t)n * 2 * sizeof(int32_t), stream);
  if (!rc && same_pool) rc = pkv_validate_copy(h, n, c);
  if (!rc && !same_pool) {
    // two pools: ids in their own pool, destinations distinct
    uint8_t* seen = (uint8_t*)calloc((size_t)dst_blocks, 1);
    if (!seen) rc = pkv__fail(PKV_EINVAL, "out of host memory");
    for (int32_t i = 0; !rc && i < n; ++i) {
      const int32_t s = h[2 * i], d = h[2 * i + 1];
      if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks)
        rc = pkv__fail(PKV_ERANGE, "pair %d = (%d, %d) outside the pools (%d, %d blocks)", i, s, d,
                       src_blocks, dst_blocks);
      else if (seen[d]++)
        rc = pkv__fail(PKV_ERANGE, "pair %d: destination block %d appears twice", i, d);
    }
    free(seen);
  }
  free(h);
  return rc;
}

}  // namespace

extern "C" int pkv_paged_kv_write(const void* k, const void* v, const int64_t* slot_mapping,
                                  int32_t num_tokens, void* k_cache, void* v_cache,
                                  const pkv_cache_desc* c, void* stream) {
  pkv__clear_error();
  int rc = pkv__check_desc(c);
  if (rc) return rc;
  if (num_tokens < 0) return pkv__fail(PKV_EINVAL, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return pkv__fail(PKV_EINVAL, "NULL device pointer");
  const int64_t row_bytes = (int64_t)c->head_dim * elem_bytes(c->dtype);
  if (row_bytes % 16 != 0)
    return pkv__fail(PKV_EUNSUPPORTED, "head_dim * element size (%lld B) is not a multiple of 16",
                     (long long)row_bytes);
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) ||
      ((uintptr_t)slot_mapping & 7u))
    return pkv__fail(PKV_EINVAL, "device pointers must be 16-byte aligned (slot_mapping 8-byte)");
  const int32_t row_chunks = (int32_t)(row_bytes / 16);
  const int64_t total = (int64_t)num_tokens * c->num_kv_heads * row_chunks;
  if (total > INT32_MAX)
    return pkv__fail(PKV_EINVAL, "write of %lld 16-byte pieces is too large (limit 2^31 - 1)",
                     (long long)total);
  if (pkv__validate_enabled()) {
    rc = validate_write_device(slot_mapping, num_tokens, c, stream);
    if (rc) return rc;
  }
  const int64_t grid = (total + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(kv_write_kernel, dim3((uint32_t)grid), dim3(kThreads), 0,
                     (hipStream_t)stream, (const uint4*)k, (const uint4*)v, slot_mapping,
                     (uint4*)k_cache, (uint4*)v_cache, (uint32_t)c->num_kv_heads,
                     (uint32_t)c->block_size, (uint32_t)row_chunks, (uint32_t)total,
                     (int64_t)c->num_blocks * c->block_size);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv__fail(PKV_EHIP, "kv_write launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

extern "C" int pkv_copy_blocks(void* k_cache, void* v_cache, const pkv_cache_desc* c,
                               const int32_t* src_dst_pairs, int32_t num_pairs, void* stream) {
  pkv__clear_error();
  int rc = pkv__check_desc(c);
  if (rc) return rc;
  if (num_pairs < 0) return pkv__fail(PKV_EINVAL, "num_pairs %d < 0", num_pairs);
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src_dst_pairs) return pkv__fail(PKV_EINVAL, "NULL device pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache) || ((uintptr_t)src_dst_pairs & 7u))
    return pkv__fail(PKV_EINVAL, "caches must be 16-byte aligned, pairs 8-byte aligned");
  const int64_t block_bytes =
      (int64_t)c->num_kv_heads * c->block_size * c->head_dim * elem_bytes(c->dtype);
  if (block_bytes % 16 != 0 || block_bytes / 16 > INT32_MAX)
    return pkv__fail(PKV_EUNSUPPORTED, "block of %lld bytes is not a multiple of 16",
                     (long long)block_bytes);
  const int32_t block_chunks = (int32_t)(block_bytes / 16);
  const int32_t groups = (block_chunks + kThreads - 1) / kThreads;
  const int64_t grid = (int64_t)num_pairs * groups;
  if (grid > INT32_MAX) return pkv__fail(PKV_EINVAL, "copy too large");
  if (pkv__validate_enabled()) {
    rc = validate_pairs_device(src_dst_pairs, num_pairs, c->num_blocks, c->num_blocks, c, true,
                               stream);
    if (rc) return rc;
  }
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((uint32_t)grid), dim3(kThreads), 0,
                     (hipStream_t)stream, (uint4*)k_cache, (uint4*)v_cache, src_dst_pairs,
                     block_chunks, groups, c->num_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv__fail(PKV_EHIP, "copy_blocks launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

extern "C" int pkv_swap_blocks(void* dst_k, void* dst_v, int32_t dst_num_blocks, const void* src_k,
                               const void* src_v, int32_t src_num_blocks, const pkv_cache_desc* c,
                               const int32_t* pairs, int32_t num_pairs, void* stream) {
  pkv__clear_error();
  if (!c) return pkv__fail(PKV_EINVAL, "cache descriptor is NULL");
  if (c->num_kv_heads <= 0 || c->block_size <= 0 || c->head_dim <= 0 ||
      (c->dtype != PKV_F32 && c->dtype != PKV_BF16))
    return pkv__fail(PKV_EINVAL, "bad block shape in the cache descriptor");
  if (dst_num_blocks <= 0 || src_num_blocks <= 0)
    return pkv__fail(PKV_EINVAL, "pool sizes must be positive (dst %d, src %d)", dst_num_blocks,
                     src_num_blocks);
  if (num_pairs < 0) return pkv__fail(PKV_EINVAL, "num_pairs %d < 0", num_pairs);
  if (num_pairs == 0) return PKV_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !pairs) return pkv__fail(PKV_EINVAL, "NULL pointer");
  if (!aligned16(dst_k) || !aligned16(dst_v) || !aligned16(src_k) || !aligned16(src_v) ||
      ((uintptr_t)pairs & 7u))
    return pkv__fail(PKV_EINVAL, "pools must be 16-byte aligned, pairs 8-byte aligned");
  const int64_t block_bytes =
      (int64_t)c->num_kv_heads * c->block_size * c->head_dim * elem_bytes(c->dtype);
  if (block_bytes % 16 != 0 || block_bytes / 16 > INT32_MAX)
    return pkv__fail(PKV_EUNSUPPORTED, "block of %lld bytes is not a multiple of 16",
                     (long long)block_bytes);
  const int32_t block_chunks = (int32_t)(block_bytes / 16);
  const int32_t groups = (block_chunks + kThreads - 1) / kThreads;
  const int64_t grid = (int64_t)num_pairs * groups;
  if (grid > INT32_MAX) return pkv__fail(PKV_EINVAL, "swap too large");
  if (pkv__validate_enabled()) {
    const int rc = validate_pairs_device(pairs, num_pairs, src_num_blocks, dst_num_blocks, c,
                                         false, stream);
    if (rc) return rc;
  }
  hipLaunchKernelGGL(swap_blocks_kernel, dim3((uint32_t)grid), dim3(kThreads), 0,
                     (hipStream_t)stream, (uint4*)dst_k, (uint4*)dst_v, dst_num_blocks,
                     (const uint4*)src_k, (const uint4*)src_v, src_num_blocks, pairs, block_chunks,
                     groups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv__fail(PKV_EHIP, "swap_blocks launch: %s", hipGetErrorString(e));
  return PKV_OK;
}
