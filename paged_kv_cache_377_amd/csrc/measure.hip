// Measurement kernel: the memory-system ceiling of the decode's access pattern.
//
// The decode's cost is the gather of K and V rows through the block table
// (weishuz.com Month 2, section 06, misconception 1: paged attention is
// ordinary attention whose K/V come from non-contiguous addresses; the
// PagedAttention blog, section 3(3): the physical blocks of a sequence are
// scattered).  This kernel reads a given list of (block, KV head) runs of both
// pools -- B x D elements of K and of V each, contiguous in the
// [block, head, token, dim] layout -- in equal contiguous shares per wave,
// with the same share rule as the balanced decode and no arithmetic but an
// XOR of the loaded words, so its time is what the memory system needs to
// deliver those bytes in that order.  It is not part of the attention path.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pagedkv_measure.h"
#include "pkv_internal.h"

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kMaxShare = 4096;  // runs per wave whose ids fit the workgroup's LDS

// PPL: 16-byte pieces of one run per lane (run bytes / 1 KiB); NBUF run
// buffers per wave (runs in flight + 1).
template <int PPL, int NBUF>
__global__ __launch_bounds__(kThreads) void gather_runs_kernel(
    const uint4* __restrict__ k_pool, const uint4* __restrict__ v_pool,
    const int32_t* __restrict__ runs, int64_t num_runs, int32_t num_workers, int32_t max_share,
    int64_t pool_runs, uint32_t* __restrict__ sink) {
  extern __shared__ int32_t sm_ids[];  // [kWaves][max_share] run ids of this workgroup's shares
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // Stage the run ids of the workgroup's shares in LDS (ids outside the pool
  // read run 0), so that no id load waits behind the run loads in flight.
  for (int wv = 0; wv < kWaves; ++wv) {
    const int ww = blockIdx.x * kWaves + wv;
    if (ww >= num_workers) break;
    const int64_t a = (int64_t)ww * num_runs / num_workers;
    const int64_t b = (int64_t)(ww + 1) * num_runs / num_workers;
    for (int64_t i = threadIdx.x; i < b - a; i += kThreads) {
      const int32_t id = runs[a + i];
      sm_ids[wv * max_share + i] = id >= 0 && id < pool_runs ? id : 0;
    }
  }
  __syncthreads();
  const int w = blockIdx.x * kWaves + wave;
  if (w >= num_workers) return;
  const int64_t u0 = (int64_t)w * num_runs / num_workers;
  const int n = (int)((int64_t)(w + 1) * num_runs / num_workers - u0);
  if (n == 0) return;
  const int32_t* ids = sm_ids + wave * max_share;

  uint4 buf[NBUF][2 * PPL];
  uint32_t acc = 0;
  // Run i of the share (a run past the share's end reads its first run again
  // and is never used); lane l reads pieces l, l + 64, ... of the run.
  auto issue = [&](int i, uint4 (&x)[2 * PPL]) {
    const int64_t r = ids[i < n ? i : 0];
    const uint4* kp = k_pool + r * (PPL * kWave) + lane;
    const uint4* vp = v_pool + r * (PPL * kWave) + lane;
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      x[p] = kp[p * kWave];
      x[PPL + p] = vp[p * kWave];
    }
  };
  auto use = [&](const uint4 (&x)[2 * PPL]) {
#pragma unroll
    for (int c = 0; c < 2 * PPL; ++c) acc ^= x[c].x ^ x[c].y ^ x[c].z ^ x[c].w;
  };
#pragma unroll
  for (int f = 0; f < NBUF - 1; ++f) issue(f, buf[f]);
  for (int i = 0; i < n; i += NBUF) {
#pragma unroll
    for (int f = 0; f < NBUF; ++f) {
      issue(i + f + NBUF - 1, buf[(f + NBUF - 1) % NBUF]);
      if (i + f < n) use(buf[f]);
    }
  }
  // every lane's words reach the stored value
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, kWave);
  if (lane == 0) sink[w] = acc;
}

template <int PPL>
int launch_ppl(const void* k, const void* v, const int32_t* runs, int64_t num_runs,
               int32_t num_workers, int32_t in_flight, int32_t max_share, int64_t pool_runs,
               uint32_t* sink, hipStream_t stream) {
  const dim3 grid((uint32_t)((num_workers + kWaves - 1) / kWaves));
  const size_t lds = (size_t)kWaves * max_share * sizeof(int32_t);
  const uint4* kp = (const uint4*)k;
  const uint4* vp = (const uint4*)v;
  switch (in_flight) {
    case 1:
      hipLaunchKernelGGL((gather_runs_kernel<PPL, 2>), grid, dim3(kThreads), lds, stream, kp, vp,
                         runs, num_runs, num_workers, max_share, pool_runs, sink);
      break;
    case 2:
      hipLaunchKernelGGL((gather_runs_kernel<PPL, 3>), grid, dim3(kThreads), lds, stream, kp, vp,
                         runs, num_runs, num_workers, max_share, pool_runs, sink);
      break;
    default:
      hipLaunchKernelGGL((gather_runs_kernel<PPL, 4>), grid, dim3(kThreads), lds, stream, kp, vp,
                         runs, num_runs, num_workers, max_share, pool_runs, sink);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv__fail(PKV_EHIP, "gather launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_measure_gather(const void* k_pool, const void* v_pool, const pkv_cache_desc* c,
                                  const int32_t* runs, int64_t num_runs, int32_t num_workers,
                                  int32_t runs_in_flight, uint32_t* sink, void* stream) {
  pkv__clear_error();
  int rc = pkv__check_desc(c);
  if (rc) return rc;
  if (num_runs < 0 || num_workers <= 0 || runs_in_flight < 1 || runs_in_flight > 3)
    return pkv__fail(PKV_EINVAL, "bad sizes (num_runs=%lld num_workers=%d runs_in_flight=%d)",
                     (long long)num_runs, num_workers, runs_in_flight);
  if (num_runs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !runs || !sink) return pkv__fail(PKV_EINVAL, "NULL pointer");
  if (((uintptr_t)k_pool | (uintptr_t)v_pool) & 15u)
    return pkv__fail(PKV_EINVAL, "pools must be 16-byte aligned");
  const int64_t max_share = (num_runs + num_workers - 1) / num_workers;
  if (max_share > kMaxShare)
    return pkv__fail(PKV_EINVAL, "%lld runs per wave; at most %d", (long long)max_share, kMaxShare);
  const int64_t run_bytes =
      (int64_t)c->block_size * c->head_dim * (c->dtype == PKV_BF16 ? 2 : 4);
  const int64_t pool_runs = (int64_t)c->num_blocks * c->num_kv_heads;
  const hipStream_t st = (hipStream_t)stream;
  switch (run_bytes) {
    case 1024: return launch_ppl<1>(k_pool, v_pool, runs, num_runs, num_workers, runs_in_flight,
                                    (int32_t)max_share, pool_runs, sink, st);
    case 2048: return launch_ppl<2>(k_pool, v_pool, runs, num_runs, num_workers, runs_in_flight,
                                    (int32_t)max_share, pool_runs, sink, st);
    case 4096: return launch_ppl<4>(k_pool, v_pool, runs, num_runs, num_workers, runs_in_flight,
                                    (int32_t)max_share, pool_runs, sink, st);
    case 8192: return launch_ppl<8>(k_pool, v_pool, runs, num_runs, num_workers, runs_in_flight,
                                    (int32_t)max_share, pool_runs, sink, st);
  }
  return pkv__fail(PKV_EUNSUPPORTED, "run of %lld bytes (built: 1, 2, 4 and 8 KiB)",
                   (long long)run_bytes);
}
