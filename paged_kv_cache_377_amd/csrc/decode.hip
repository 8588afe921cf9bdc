// Paged decode attention for gfx950: split-context partitions + reduce.
//
// What is computed (PagedAttention blog, 0539edu.com, section 3(3), step 2;
// weishuz.com Month 2, section 06, misconception 1): ordinary softmax
// attention of one query token per sequence over that sequence's cached
// tokens, whose K/V rows are gathered from scattered physical blocks through
// the block table.  The table lives in GPU memory and is read inside the
// kernel (weishuz.com Month 2, section 02, row "TLB").
//
// Work decomposition.  One workgroup (4 waves of 64 lanes) per (sequence,
// KV head, partition of `ps` tokens).  The query heads sharing the KV head
// (the group of G = Hq / Hkv heads) are processed together, so each K/V byte
// is read from HBM once per step.  Wave w walks blocks w, w+4, ... of its
// partition with an online softmax; the four waves merge through LDS.  A
// sequence that fits one partition writes its output directly; otherwise
// each partition writes (max, sum, unnormalised output) and a small reduce
// kernel combines them.
//
// Lane layout.  A (block, head) run is block_size rows of head_dim elements.
// Each lane loads 16 bytes (EPL elements) of a row; LPT = head_dim / EPL
// lanes cover one token row and one wave load covers TPL = 64 / LPT tokens
// (1 KiB, contiguous).  Dot products are summed over the LPT lanes of a
// token with DPP row operations; the token's softmax weight is then already
// in every lane that holds a piece of its V row, and the P*V products
// accumulate per lane with no exchange until the end of the partition.
//
// Numerics: fp32 throughout, logits in the base-2 domain (q is pre-scaled by
// scale * log2 e, exponentials are exp2), output rounded to the cache dtype
// (bf16: round-to-nearest-even).  Masked tokens are selected out, never
// multiplied by zero, so NaN bits in unfilled slots cannot reach the result.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

struct F32 {
  using raw = float;
  static constexpr int bytes = 4;
};
struct BF16 {
  using raw = uint16_t;
  static constexpr int bytes = 2;
};

// ---------------------------------------------------------------- helpers

__device__ inline void unpack(const uint4& x, float (&f)[4]) {
  f[0] = __uint_as_float(x.x);
  f[1] = __uint_as_float(x.y);
  f[2] = __uint_as_float(x.z);
  f[3] = __uint_as_float(x.w);
}

__device__ inline void unpack(const uint4& x, float (&f)[8]) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ inline uint16_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ inline void store_out(float* p, float x) { *p = x; }
__device__ inline void store_out(uint16_t* p, float x) { *p = f32_to_bf16_rne(x); }

template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

__device__ inline float xor16(float x) {
  // ds_swizzle bitmask mode: and 0x1f, or 0, xor 0x10 (within 32 lanes)
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401f));
}

__device__ inline float xor32(float x) { return __shfl_xor(x, 32, kWave); }

// Sum over aligned groups of N lanes; every lane of a group gets the same
// bits (each step adds two equal partial sums in either order).
template <int N>
__device__ inline float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xb1>(x);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp<0x4e>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror
  if constexpr (N >= 32) x += xor16(x);
  if constexpr (N >= 64) x += xor32(x);
  return x;
}

// Reduce over lanes l with equal l % N (across the 64 / N groups), for
// values that differ per lane.
template <int N>
__device__ inline float across_sum(float x) {
  if constexpr (N <= 8) x += dpp<0x128>(x);  // row_ror:8 == lane xor 8
  if constexpr (N <= 16) x += xor16(x);
  if constexpr (N <= 32) x += xor32(x);
  return x;
}

template <int N>
__device__ inline float across_max(float x) {
  if constexpr (N <= 8) x = fmaxf(x, dpp<0x128>(x));
  if constexpr (N <= 16) x = fmaxf(x, xor16(x));
  if constexpr (N <= 32) x = fmaxf(x, xor32(x));
  return x;
}

// ------------------------------------------------------------ partition

// Workspace layout for P > 1:
//   part_ml [S][Hq][P][2] f32  (running max in log2 units, sum of weights)
//   part_o  [S][Hq][P][D] f32  (unnormalised weighted sum of V)
template <typename E, int D, int B, int G>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(
    const typename E::raw* __restrict__ q, const uint4* __restrict__ k_cache,
    const uint4* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    int32_t table_width, const int32_t* __restrict__ context_lens,
    typename E::raw* __restrict__ out, float* __restrict__ part_ml,
    float* __restrict__ part_o, int32_t num_kv_heads, int32_t num_blocks, int32_t num_parts,
    int32_t ps, int32_t max_context_len, float qscale) {
  constexpr int EPL = 16 / E::bytes;  // elements per lane load
  constexpr int LPT = D / EPL;        // lanes per token row
  constexpr int TPL = kWave / LPT;    // tokens per wave load
  constexpr int LPB = B / TPL;        // wave loads per block
  static_assert(LPT >= 8 && LPT <= 32 && LPB >= 1 && LPB * TPL == B, "unsupported shape");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int p = blockIdx.x % num_parts;
  const int sg = blockIdx.x / num_parts;
  const int g = sg % num_kv_heads;
  const int s = sg / num_kv_heads;
  const int hq = num_kv_heads * G;
  // Lengths outside [0, max_context_len] break the caller's contract; clamping
  // keeps every table, cache and workspace access in bounds regardless.
  const int n = min(max(context_lens[s], 0), max_context_len);
  const int t0 = p * ps;

  if (n == 0) {
    if (p != 0) return;
    for (int i = threadIdx.x; i < G * D; i += kThreads)
      store_out(out + ((int64_t)s * hq + g * G) * D + i, 0.0f);
    return;
  }
  if (t0 >= n) return;  // partition past the end of this sequence
  const int t1 = min(n, t0 + ps);
  const int b0 = t0 / B;
  const int b1 = (t1 + B - 1) / B;
  const int nparts_s = (n + ps - 1) / ps;

  const int c = lane % LPT;  // which 16-byte piece of a row
  const int r = lane / LPT;  // which token of a wave load

  // This lane's piece of the G query rows, scaled into log2 units.
  float qr[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 raw = *reinterpret_cast<const uint4*>(q + ((int64_t)s * hq + g * G + h) * D +
                                                      c * EPL);
    unpack(raw, qr[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qr[h][e] *= qscale;
  }

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
  }

  const int32_t* bt = block_tables + (int64_t)s * table_width;
  constexpr int RUN = B * LPT;  // 16-byte pieces per (block, head) run

  for (int b = b0 + wave; b < b1; b += kWaves) {
    int64_t phys = bt[b];
    // An id outside the pool breaks the caller's contract: its tokens are
    // dropped instead of being read out of bounds.
    const bool in_pool = phys >= 0 && phys < num_blocks;
    if (!in_pool) phys = 0;
    const uint4* kb = k_cache + (phys * num_kv_heads + g) * RUN;
    const uint4* vb = v_cache + (phys * num_kv_heads + g) * RUN;
    uint4 kr[LPB], vr[LPB];
#pragma unroll
    for (int j = 0; j < LPB; ++j) {
      kr[j] = kb[(j * TPL + r) * LPT + c];
      vr[j] = vb[(j * TPL + r) * LPT + c];
    }
    const bool full = in_pool && (b + 1) * B <= n;  // same for the whole wave
    bool valid[LPB];
#pragma unroll
    for (int j = 0; j < LPB; ++j) valid[j] = true;

    float sc[LPB][G];
#pragma unroll
    for (int j = 0; j < LPB; ++j) {
      float kf[EPL];
      unpack(kr[j], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) a = fmaf(qr[h][e], kf[e], a);
        sc[j][h] = group_sum<LPT>(a);
      }
    }
    if (!full) {
#pragma unroll
      for (int j = 0; j < LPB; ++j) {
        valid[j] = in_pool && b * B + j * TPL + r < n;
#pragma unroll
        for (int h = 0; h < G; ++h) sc[j][h] = valid[j] ? sc[j][h] : -INFINITY;
        if (!valid[j]) vr[j] = make_uint4(0, 0, 0, 0);
      }
    }

#pragma unroll
    for (int h = 0; h < G; ++h) {
      float bm = sc[0][h];
#pragma unroll
      for (int j = 1; j < LPB; ++j) bm = fmaxf(bm, sc[j][h]);
      bm = across_max<LPT>(bm);
      if (bm > m[h]) {  // wave-uniform
        const float alpha = exp2f(m[h] - bm);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
        m[h] = bm;
      }
    }

#pragma unroll
    for (int j = 0; j < LPB; ++j) {
      float vf[EPL];
      unpack(vr[j], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        // masked tokens weigh exactly 0 (even before any valid token set m)
        const float pw = valid[j] ? exp2f(sc[j][h] - m[h]) : 0.0f;
        l[h] += pw;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pw, vf[e], acc[h][e]);
      }
    }
  }

  // Combine the token groups of this wave: lanes with equal c.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = across_sum<LPT>(l[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = across_sum<LPT>(acc[h][e]);
  }

  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  __shared__ float sm_o[kWaves][G][D];
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm_m[wave][h] = m[h];
      sm_l[wave][h] = l[h];
    }
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[wave][h][c * EPL + e] = acc[h][e];
  }
  __syncthreads();

  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int h = i / D;
    const int d = i - h * D;
    float mx = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm_m[w][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      // a wave that saw no block has m = -inf and contributes nothing
      const float f = sm_m[w][h] == -INFINITY ? 0.0f : exp2f(sm_m[w][h] - mx);
      L = fmaf(sm_l[w][h], f, L);
      O = fmaf(sm_o[w][h][d], f, O);
    }
    const int64_t row = (int64_t)s * hq + g * G + h;
    if (nparts_s == 1) {
      store_out(out + row * D + d, O / L);
    } else {
      part_o[(row * num_parts + p) * D + d] = O;
      if (d == 0) {
        part_ml[(row * num_parts + p) * 2 + 0] = mx;
        part_ml[(row * num_parts + p) * 2 + 1] = L;
      }
    }
  }
}

// --------------------------------------------------------------- reduce

// One workgroup of D threads per (sequence, query head) whose sequence spans
// more than one partition: out = sum_p o_p 2^(m_p - m*) / sum_p L_p 2^(m_p - m*).
template <typename E, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(
    typename E::raw* __restrict__ out, const float* __restrict__ part_ml,
    const float* __restrict__ part_o, const int32_t* __restrict__ context_lens,
    int32_t num_q_heads, int32_t num_parts, int32_t ps, int32_t max_context_len) {
  const int h = blockIdx.x % num_q_heads;
  const int s = blockIdx.x / num_q_heads;
  const int n = min(max(context_lens[s], 0), max_context_len);
  const int np = (n + ps - 1) / ps;
  if (np <= 1) return;
  const int d = threadIdx.x;
  const int64_t row = (int64_t)s * num_q_heads + h;
  const float* ml = part_ml + row * num_parts * 2;
  float mx = -INFINITY;
  for (int p = 0; p < np; ++p) mx = fmaxf(mx, ml[2 * p]);
  float L = 0.0f, O = 0.0f;
  for (int p = 0; p < np; ++p) {
    const float f = exp2f(ml[2 * p] - mx);
    L = fmaf(ml[2 * p + 1], f, L);
    O = fmaf(part_o[(row * num_parts + p) * D + d], f, O);
  }
  store_out(out + row * D + d, O / L);
}

// ------------------------------------------------------------- dispatch

struct LaunchArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int32_t width;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t max_context_len;
  int32_t num_q_heads;
  int32_t num_parts;
  int32_t ps;
  float qscale;
  float* part_ml;
  float* part_o;
  hipStream_t stream;
};

template <typename E, int D, int B, int G>
int launch(const LaunchArgs& a) {
  const int64_t grid = (int64_t)a.num_seqs * a.num_kv_heads * a.num_parts;
  if (grid > INT32_MAX) return pkv__fail(PKV_EINVAL, "decode grid too large");
  hipLaunchKernelGGL((decode_partition_kernel<E, D, B, G>), dim3((uint32_t)grid),
                     dim3(kThreads), 0, a.stream, (const typename E::raw*)a.q,
                     (const uint4*)a.k_cache, (const uint4*)a.v_cache, a.block_tables,
                     a.width, a.context_lens, (typename E::raw*)a.out, a.part_ml, a.part_o,
                     a.num_kv_heads, a.num_blocks, a.num_parts, a.ps, a.max_context_len,
                     a.qscale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv__fail(PKV_EHIP, "decode_partition launch: %s", hipGetErrorString(e));
  if (a.num_parts > 1) {
    hipLaunchKernelGGL((decode_reduce_kernel<E, D>), dim3((uint32_t)(a.num_seqs * a.num_q_heads)),
                       dim3(D), 0, a.stream, (typename E::raw*)a.out, a.part_ml, a.part_o,
                       a.context_lens, a.num_q_heads, a.num_parts, a.ps, a.max_context_len);
    e = hipGetLastError();
    if (e != hipSuccess) return pkv__fail(PKV_EHIP, "decode_reduce launch: %s", hipGetErrorString(e));
  }
  return PKV_OK;
}

template <typename E, int D, int B>
int dispatch_g(const LaunchArgs& a, int G) {
  switch (G) {
    case 1: return launch<E, D, B, 1>(a);
    case 2: return launch<E, D, B, 2>(a);
    case 4: return launch<E, D, B, 4>(a);
    case 8: return launch<E, D, B, 8>(a);
  }
  return pkv__fail(PKV_EUNSUPPORTED, "query heads per KV head = %d (compiled: 1, 2, 4, 8)", G);
}

template <typename E, int D>
int dispatch_b(const LaunchArgs& a, int B, int G) {
  switch (B) {
    case 8: return dispatch_g<E, D, 8>(a, G);
    case 16: return dispatch_g<E, D, 16>(a, G);
    case 32: return dispatch_g<E, D, 32>(a, G);
  }
  return pkv__fail(PKV_EUNSUPPORTED, "block_size %d (compiled: 8, 16, 32)", B);
}

template <typename E>
int dispatch_d(const LaunchArgs& a, int D, int B, int G) {
  switch (D) {
    case 64: return dispatch_b<E, 64>(a, B, G);
    case 128: return dispatch_b<E, 128>(a, B, G);
  }
  return pkv__fail(PKV_EUNSUPPORTED, "head_dim %d (compiled: 64, 128)", D);
}

int32_t parts_for(int32_t max_context_len, int32_t partition_size) {
  if (partition_size <= 0 || max_context_len <= 0) return 1;
  return (max_context_len + partition_size - 1) / partition_size;
}

size_t workspace_for(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t parts) {
  if (parts <= 1) return 0;
  return (size_t)num_seqs * num_q_heads * parts * (2 + head_dim) * sizeof(float);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t head_dim, int32_t max_context_len,
                                             int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  return workspace_for(num_seqs, num_q_heads, head_dim,
                       parts_for(max_context_len, partition_size));
}

extern "C" int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                                          const void* v_cache, const pkv_cache_desc* c,
                                          const int32_t* block_tables,
                                          int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_q_heads, int32_t max_context_len,
                                          float scale, int32_t partition_size, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  pkv__clear_error();
  int rc = pkv__check_desc(c);
  if (rc) return rc;
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || max_blocks_per_seq < 0)
    return pkv__fail(PKV_EINVAL, "bad sizes (num_seqs=%d num_q_heads=%d max_context_len=%d width=%d)",
                     num_seqs, num_q_heads, max_context_len, max_blocks_per_seq);
  if (num_q_heads % c->num_kv_heads != 0)
    return pkv__fail(PKV_EINVAL, "num_q_heads %d is not a multiple of num_kv_heads %d",
                     num_q_heads, c->num_kv_heads);
  const int32_t B = c->block_size;
  if ((int64_t)max_blocks_per_seq * B < max_context_len)
    return pkv__fail(PKV_EINVAL, "table width %d * block_size %d < max_context_len %d",
                     max_blocks_per_seq, B, max_context_len);
  if (partition_size < 0 || (partition_size > 0 && partition_size % B != 0))
    return pkv__fail(PKV_EINVAL, "partition_size %d must be 0 or a positive multiple of block_size %d",
                     partition_size, B);
  if (!(scale == scale) || isinf(scale)) return pkv__fail(PKV_EINVAL, "scale is not finite");
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return pkv__fail(PKV_EINVAL, "NULL device pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      ((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u))
    return pkv__fail(PKV_EINVAL, "q, out and caches must be 16-byte aligned");

  const int32_t parts = parts_for(max_context_len, partition_size);
  // With no split, one partition holds the longest context.
  const int32_t ps = parts == 1 ? (max_context_len > 0 ? ((max_context_len + B - 1) / B) * B : B)
                                : partition_size;
  const size_t need = workspace_for(num_seqs, num_q_heads, c->head_dim, parts);
  if (workspace_bytes < need || (need && !workspace))
    return pkv__fail(PKV_EINVAL, "workspace of %zu bytes is smaller than the %zu needed",
                     workspace_bytes, need);
  if (need && !aligned16(workspace)) return pkv__fail(PKV_EINVAL, "workspace must be 16-byte aligned");

  LaunchArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.width = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_kv_heads = c->num_kv_heads;
  a.num_blocks = c->num_blocks;
  a.max_context_len = max_context_len;
  a.num_q_heads = num_q_heads;
  a.num_parts = parts;
  a.ps = ps;
  a.qscale = scale * kLog2e;
  a.part_ml = need ? (float*)workspace : nullptr;
  a.part_o = need ? (float*)workspace + (size_t)num_seqs * num_q_heads * parts * 2 : nullptr;
  a.stream = (hipStream_t)stream;
  const int G = num_q_heads / c->num_kv_heads;
  if (c->dtype == PKV_BF16) return dispatch_d<BF16>(a, c->head_dim, B, G);
  return dispatch_d<F32>(a, c->head_dim, B, G);
}
