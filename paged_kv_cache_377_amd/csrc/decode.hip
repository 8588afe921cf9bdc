// Paged decode attention for gfx950: split-context partitions + reduce.
//
// What is computed (PagedAttention blog, 0539edu.com, section 3(3), step 2;
// weishuz.com Month 2, section 06, misconception 1): ordinary softmax
// attention of one query token per sequence over that sequence's cached
// tokens, whose K/V rows are gathered from scattered physical blocks through
// the block table.  The table lives in GPU memory and is read inside the
// kernel (weishuz.com Month 2, section 02, row "TLB").
//
// Work decomposition (both kernels).  One workgroup (4 waves of 64 lanes) per
// (sequence, KV head, partition of `ps` tokens).  The query heads sharing the
// KV head (the group of G = Hq / Hkv heads) are processed together, so each
// K/V byte is read from HBM once per step.  Each wave keeps an online softmax
// over its share of the partition; the four waves merge through LDS.  A
// sequence that fits one partition writes its output directly; otherwise each
// partition writes (max, sum, unnormalised output) and a small reduce kernel
// combines them.
//
// bf16 caches: decode_partition_mfma_kernel.  The per-token work is two small
// dense contractions (scores = K q^T, output = P V), run on the matrix cores
// (v_mfma_f32_16x16x32_bf16) over tiles of 16 tokens:
//   * scores: A = 16 K rows (tokens), B = the group's query rows (columns =
//     heads, zero-padded to 16);
//   * V^T: V is stored token-major, but the output product contracts over
//     tokens, so each 16x16 tile of V is transposed by multiplying the 16 V
//     rows with a 0/1 selection matrix (exact: one non-zero term per output);
//   * output: A = V^T tile (rows = 16 dims), B = P (columns = heads), with P
//     split into a bf16 high part and a bf16 low part (both in the contraction)
//     so the weights keep ~16 significant bits.
// The output tile of a head lands in the lanes that hold that head's softmax
// statistics, so rescaling needs no data exchange.  The running maximum is
// only moved when a tile's maximum exceeds it by more than 2^8 (log2 units),
// which keeps every weight <= 2^8 and makes rescales rare.
//
// fp32 caches: decode_partition_valu_kernel.  Each lane loads 16 bytes of a
// K/V row; dot products are summed over the lanes of a row with DPP row
// operations and P*V accumulates per lane in fp32 FMAs.
//
// Numerics: fp32 accumulation, logits in the base-2 domain (scale * log2 e),
// exponentials are exp2, output rounded to the cache dtype (bf16:
// round-to-nearest-even).  Masked tokens are selected out, never multiplied
// by zero, so NaN bits in unfilled slots cannot reach the result.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdlib.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "pagedkv_measure.h"
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

// Maximum over aligned groups of N lanes; every lane of a group gets it.
template <int N>
__device__ inline float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<0xb1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<0x4e>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<0x141>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<0x140>(x));
  if constexpr (N >= 32) x = fmaxf(x, xor16(x));
  if constexpr (N >= 64) x = fmaxf(x, xor32(x));
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
//   part_ml [S][Hq][P][2] f32  (reference max in log2 units, sum of weights)
//   part_o  [S][Hq][P][D] f32  (unnormalised weighted sum of V)
//
// Combine the four waves' (m, l, o) of one workgroup, held in LDS, and write
// either the final output row (the sequence has one partition) or this
// partition's partial.  Must be called by all kThreads threads after a barrier.
template <typename T, int D, int G>
__device__ inline void merge_waves(const float (&sm_m)[kWaves][G], const float (&sm_l)[kWaves][G],
                                   const float (&sm_o)[kWaves][G][D], int64_t row0, int p,
                                   int num_parts, int nparts_s, T* __restrict__ out,
                                   float* __restrict__ part_ml, float* __restrict__ part_o) {
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int h = i / D;
    const int d = i - h * D;
    float mx = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm_m[w][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      // a wave that saw no token has m = -inf and contributes nothing
      const float f = sm_m[w][h] == -INFINITY ? 0.0f : exp2f(sm_m[w][h] - mx);
      L = fmaf(sm_l[w][h], f, L);
      O = fmaf(sm_o[w][h][d], f, O);
    }
    const int64_t row = row0 + h;
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

template <typename E, int D, int B, int G>
__global__ __launch_bounds__(kThreads) void decode_partition_valu_kernel(
    const typename E::raw* __restrict__ q, const uint4* __restrict__ k_cache,
    const uint4* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    int32_t table_width, const int32_t* __restrict__ context_lens,
    typename E::raw* __restrict__ out, float* __restrict__ part_ml,
    float* __restrict__ part_o, int32_t num_seqs, int32_t num_kv_heads, int32_t num_blocks,
    int32_t num_parts, int32_t ps, int32_t max_context_len, float qscale) {
  constexpr int EPL = 16 / E::bytes;  // elements per lane load
  constexpr int LPT = D / EPL;        // lanes per token row
  constexpr int TPL = kWave / LPT;    // tokens per wave load
  constexpr int LPB = B / TPL;        // wave loads per block
  static_assert(LPT >= 8 && LPT <= 32 && LPB >= 1 && LPB * TPL == B, "unsupported shape");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // Grid order (partition, sequence, KV head), KV head fastest: workgroups
  // are dealt round-robin to the XCDs, so consecutive ids must carry similar
  // work.  With the partition fastest, every sequence's partition 0 (always
  // present) would land on one XCD and its late, mostly empty partitions on
  // another.
  const int g = blockIdx.x % num_kv_heads;
  const int ps_idx = blockIdx.x / num_kv_heads;
  const int s = ps_idx % num_seqs;
  const int p = ps_idx / num_seqs;
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

  merge_waves<typename E::raw, D, G>(sm_m, sm_l, sm_o, (int64_t)s * hq + g * G, p, num_parts,
                                    nparts_s, out, part_ml, part_o);
}

// ------------------------------------------------------------ MFMA (bf16)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;  // tokens per MFMA tile

// D = A B + C on a 16x16x32 bf16 tile.  Lane l supplies row (l % 16) of A and
// column (l % 16) of B, each as 8 consecutive k-slots of group l / 16; it
// receives D[4 (l / 16) + r][l % 16] in element r.  Only the pairing of A's
// and B's k-slots matters to the kernels, not their order.
__device__ inline f32x4_t mfma16x16x32(const uint4& a, const uint4& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Two fp32 values that are exactly bf16 numbers -> one packed bf16 pair.
__device__ inline uint32_t pack_bf16_pair(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum over the four 16-lane rows of the wave (lanes with equal l % 16),
// with the VALU row-swap instructions: after a swap each lane holds its own
// value and its partner row's value in the two results.
__device__ inline float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ inline float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// A tile's maximum must exceed the reference maximum by more than this (log2
// units) before the accumulators are rescaled; weights stay <= 2^8.
constexpr float kRescaleSlack = 8.0f;

// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their
// maxima (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
constexpr int kWaitVmcnt0 = (7 << 4) | (15 << 8);

// The K and V pieces of the 16 token rows of one tile as one wave holds them:
// lane (grp = l / 16, col = l % 16) has dims 32 kk + 8 grp .. + 7 of row col.
template <int D>
struct KVTile {
  uint4 k[D / 32], v[D / 32];
  bool ok;  // this lane's row is live and its block id is inside the pool
};

// Load row `tok` (offset tok % B of block `phys`, KV head g) into x.  A row
// that is not live, or whose block id is outside the pool, reads `safe` (a
// small in-bounds row) instead, and its V is zeroed when it is used.  The
// loads are never predicated, so the compiler can count them in flight.
// A non-null k_row / v_row replaces the cache as the source of the row (the
// appended token of the fused append + decode, read from its input).
template <int D, int B>
__device__ inline void load_kv(KVTile<D>& x, const uint16_t* __restrict__ k_cache,
                               const uint16_t* __restrict__ v_cache, const uint16_t* safe,
                               bool live, int phys, int tok, int g, int num_kv_heads,
                               int num_blocks, int grp, const uint16_t* k_row = nullptr,
                               const uint16_t* v_row = nullptr) {
  x.ok = live && phys >= 0 && phys < num_blocks;
  const int64_t off = ((int64_t)phys * num_kv_heads + g) * (B * D) + (int64_t)(tok % B) * D + 8 * grp;
  const uint16_t* kp = x.ok ? (k_row ? k_row : k_cache + off) : safe;
  const uint16_t* vp = x.ok ? (v_row ? v_row : v_cache + off) : safe;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    x.k[kk] = *reinterpret_cast<const uint4*>(kp + 32 * kk);
    x.v[kk] = *reinterpret_cast<const uint4*>(vp + 32 * kk);
  }
}

// One wave's online-softmax state for the G query heads of one KV head and its
// update by one tile on the matrix cores (v_mfma_f32_16x16x32_bf16):
//   * scores: A = the 16 K rows (tokens), B = the group's query rows (columns
//     = heads, zero past G); lane (grp, col) receives the scores of tokens
//     4 grp + r for head col;
//   * V^T: V is token-major but the output product contracts over tokens, so
//     each 16x16 tile of V is transposed by a product with a 0/1 selection
//     matrix (exact: one non-zero term per output);
//   * output: A = V^T tile (rows = 16 dims), B = P (columns = heads) with P
//     split into a bf16 high part and a bf16 low part (both in the contraction)
//     so the weights keep ~16 significant bits.
// The output tile of a head lands in the lanes that hold that head's softmax
// statistics, so rescaling needs no data exchange.
template <int D, int G>
struct MfmaAttn {
  static constexpr int KP = D / 32;  // 32-dim pieces of a row
  static constexpr int DT = D / 16;  // 16-dim output tiles
  static_assert(D % 32 == 0 && G >= 1 && G <= 16, "unsupported shape");
  uint4 qb[KP];   // B operand of the scores: q[head col][dims 32 kk + 8 grp ..]
  uint4 sel[2];   // selection matrices of the V transposes
  f32x4_t o[DT];  // o[j][r] = unnormalised output, head col, dim 16 j + 4 grp + r
  float m;        // reference maximum of head col (log2 units)
  float l;        // this lane's share of the weight sum of head col

  __device__ void init(int col, int grp) {
    // column c of half h picks dim 16 h + c of a 32-dim piece, i.e. k-slot
    // (2 h + c / 8, c % 8).  bf16 1.0 = 0x3f80.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool on = grp == 2 * h + (col >> 3);
      const int e = col & 7;
      const uint32_t one = 0x3f80u << (16 * (e & 1));
      sel[h] = make_uint4(on && (e >> 1) == 0 ? one : 0u, on && (e >> 1) == 1 ? one : 0u,
                          on && (e >> 1) == 2 ? one : 0u, on && (e >> 1) == 3 ? one : 0u);
    }
    reset();
  }

  __device__ void reset() {
#pragma unroll
    for (int j = 0; j < DT; ++j) o[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m = -INFINITY;
    l = 0.0f;
  }

  // qgroup = q row of the group's first head.  k-slot (grp, e) of piece kk is
  // dim 32 kk + 8 grp + e for K rows and q alike.  Columns past the group's G
  // heads are zero (their lanes read the first head's row).
  __device__ void load_q(const uint16_t* qgroup, int col, int grp) {
    const uint16_t* qrow = qgroup + (col < G ? col : 0) * D + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < KP; ++kk) {
      const uint4 x = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
      qb[kk] = col < G ? x : make_uint4(0, 0, 0, 0);
    }
  }

  // Rows 0 .. nvalid - 1 of the tile count (1 <= nvalid <= 16); later rows
  // are masked, whatever their K and V bits.
  __device__ void update(KVTile<D>& x, int nvalid, float qscale, int grp) {
    // V rows that do not count become zeros (their weight is 0, and 0 * NaN
    // would otherwise poison the output)
#pragma unroll
    for (int kk = 0; kk < KP; ++kk)
      if (!x.ok) x.v[kk] = make_uint4(0, 0, 0, 0);
    // V^T tiles first: they do not depend on the scores, so these products
    // overlap the score products and the softmax arithmetic.
    // va[j] = bf16 pairs of V[token 4 grp + r][dim 16 j + col], r = 0..3
    uint32_t va[DT][2];
#pragma unroll
    for (int j = 0; j < DT; ++j) {
      const f32x4_t tv = mfma16x16x32(x.v[j >> 1], sel[j & 1], f32x4_t{0.0f, 0.0f, 0.0f, 0.0f});
      va[j][0] = pack_bf16_pair(tv[0], tv[1]);
      va[j][1] = pack_bf16_pair(tv[2], tv[3]);
    }
    f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KP; ++kk) sc = mfma16x16x32(x.k[kk], qb[kk], sc);
    float sv[4];
    float bm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = 4 * grp + r < nvalid ? sc[r] * qscale : -INFINITY;
      bm = fmaxf(bm, sv[r]);
    }
    bm = rows_max(bm);  // maximum over the tile's tokens
    const bool need = bm > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float alpha = need ? fast_exp2(m - bm) : 1.0f;  // 0 on the first tile
      m = need ? bm : m;
      l *= alpha;
#pragma unroll
      for (int j = 0; j < DT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[j][r] *= alpha;
    }
    float pw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pw[r] = fast_exp2(sv[r] - m);  // masked rows: exactly 0
    l += (pw[0] + pw[1]) + (pw[2] + pw[3]);
    // P as the B operand: k-slots e < 4 hold the bf16 high parts of the
    // weights of tokens 4 grp + e, slots e >= 4 the rounded remainders.
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      hi[r] = __float_as_uint(pw[r]) & 0xffff0000u;
      lo[r] = (__float_as_uint(pw[r] - __uint_as_float(hi[r])) + 0x8000u) & 0xffff0000u;
    }
    const uint4 pb = make_uint4((hi[0] >> 16) | hi[1], (hi[2] >> 16) | hi[3],
                                (lo[0] >> 16) | lo[1], (lo[2] >> 16) | lo[3]);
    // o[j] element r += sum_t V[t][dim 16 j + 4 grp + r] * P[t][head col]
#pragma unroll
    for (int j = 0; j < DT; ++j)
      o[j] = mfma16x16x32(make_uint4(va[j][0], va[j][1], va[j][0], va[j][1]), pb, o[j]);
  }
};

// Split-context kernel for bf16 caches: one workgroup per (partition,
// sequence, KV head), block-table entries of the partition staged in LDS.
template <int D, int B, int G>
__global__ __launch_bounds__(kThreads) void decode_partition_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    int32_t table_width, const int32_t* __restrict__ context_lens, uint16_t* __restrict__ out,
    float* __restrict__ part_ml, float* __restrict__ part_o, int32_t num_seqs,
    int32_t num_kv_heads, int32_t num_blocks, int32_t num_parts, int32_t ps,
    int32_t max_context_len, float qscale) {
  constexpr int DT = D / 16;
  constexpr int kChunkTiles = 64;      // tiles whose table entries are staged at once
  constexpr int kChunkEntries = kChunkTiles * kTile / B + 2;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int col = lane & 15;  // token row of the loads; head column of scores and outputs
  const int grp = lane >> 4;  // k-slot group of the operands; row group of the results
  // Grid order (partition, sequence, KV head), KV head fastest: workgroups
  // are dealt round-robin to the XCDs, so consecutive ids must carry similar
  // work.  With the partition fastest, every sequence's partition 0 (always
  // present) would land on one XCD and its late, mostly empty partitions on
  // another.
  const int g = blockIdx.x % num_kv_heads;
  const int ps_idx = blockIdx.x / num_kv_heads;
  const int s = ps_idx % num_seqs;
  const int p = ps_idx / num_seqs;
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
  const int ntiles = (t1 - t0 + kTile - 1) / kTile;
  const int nparts_s = (n + ps - 1) / ps;

  MfmaAttn<D, G> at;
  at.init(col, grp);
  at.load_q(q + ((int64_t)s * hq + g * G) * D, col, grp);

  __shared__ int32_t sm_bt[kChunkEntries];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  __shared__ float sm_o[kWaves][G][D];

  const int32_t* bt = block_tables + (int64_t)s * table_width;
  const uint16_t* safe = q + 8 * grp;

  // A live row of the chunk [c0, c1) lies at or before the chunk's last
  // position `last`; a dead row (tile -1 or past t1) reads the table entry of
  // `last`, so the LDS index stays below the chunk's staged entry count.
  auto load_tile = [&](int tile, int cb0, int last, KVTile<D>& x) {
    const int t = t0 + tile * kTile + col;
    const bool live = tile >= 0 && t < t1;
    const int tc = live ? t : last;
    load_kv<D, B>(x, k_cache, v_cache, safe, live, sm_bt[tc / B - cb0], tc, g, num_kv_heads,
                  num_blocks, grp);
  };

  for (int c0 = 0; c0 < ntiles; c0 += kChunkTiles) {
    const int c1 = min(ntiles, c0 + kChunkTiles);
    const int cb0 = (t0 + c0 * kTile) / B;
    const int cb1 = (min(t1, t0 + c1 * kTile) - 1) / B + 1;
    __syncthreads();  // the previous chunk's entries are no longer read
    for (int i = threadIdx.x; i < cb1 - cb0; i += kThreads) sm_bt[i] = bt[cb0 + i];
    __syncthreads();
    int tile = c0 + wave;
    if (tile >= c1) continue;
    // Nothing but the tile loads below may be in flight when the loop is
    // entered, so the compiler can count them precisely (vmcnt) in the loop.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    // Two tile buffers in turn: the loads of the next tile (or of dummy rows)
    // are issued before the current tile is processed.  The wave's tile count
    // is padded to an even number so the loop has a single exit, which keeps
    // the compiler's load counting exact across the back edge.
    const int mine = (c1 - 1 - tile) / kWaves + 1;
    const int last = min(t1, t0 + c1 * kTile) - 1;  // the chunk's last position
    KVTile<D> ta, tb;
    load_tile(tile, cb0, last, ta);
    for (int it = 0; it < (mine + 1) / 2; ++it, tile += 2 * kWaves) {
      const int t_b = tile + kWaves;
      const int t_c = tile + 2 * kWaves;
      load_tile(t_b < c1 ? t_b : -1, cb0, last, tb);
      at.update(ta, min(kTile, t1 - (t0 + tile * kTile)), qscale, grp);
      load_tile(t_c < c1 ? t_c : -1, cb0, last, ta);
      if (t_b < c1) at.update(tb, min(kTile, t1 - (t0 + t_b * kTile)), qscale, grp);
    }
  }

  // the four row groups of a head hold disjoint tokens' weight sums
  const float l = rows_sum(at.l);
  if (grp == 0 && col < G) {
    sm_m[wave][col] = at.m;
    sm_l[wave][col] = l;
  }
  if (col < G) {
#pragma unroll
    for (int j = 0; j < DT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm_o[wave][col][16 * j + 4 * grp + r] = at.o[j][r];
  }
  __syncthreads();
  merge_waves<uint16_t, D, G>(sm_m, sm_l, sm_o, (int64_t)s * hq + g * G, p, num_parts, nparts_s,
                              out, part_ml, part_o);
}

// ------------------------------------------------------ balanced (bf16)
//
// The work is the list of all 16-token tiles of all sequences, numbered
// sequence by sequence.  A group of gs waves (gs KV heads of one sequence,
// one head per wave; the heads are cut into Hkv / gs chunks) is a worker
// that takes one contiguous, equal share [j T / ng, (j + 1) T / ng) of the
// T = (Hkv / gs) x (tiles of all sequences) (sequence, chunk, tile) items,
// so every worker reads the same number of K/V bytes however ragged the
// context lengths are, and streams its share with the next tiles' loads
// always in flight.  The waves of a group walk the same tiles side by side,
// so the gs head runs of one block, which sit next to each other in the
// [block, head, token, dim] layout (32 KiB of K and of V for 8 heads of 16
// tokens x 128 dims), are requested together: a random gather of such runs
// streams faster than one of separate 4 KiB runs.  ng = min(T, the groups
// the GPU holds at once).
// A worker's share cuts the (sequence, chunk) list into segments; for each
// segment every wave of the group either writes its head's finished output
// (the group holds the whole sequence) or a partial (m, l, o) to slot
// ((sequence x chunks + chunk + j) gs + wave in group), and the group holding
// a sequence's first tile records which groups cover it (every record is
// rewritten on every call: empty sequences' pairs are marked by the
// workgroups).  Slots are distinct: along the item list, sequence x chunks +
// chunk + j grows by at least one at every segment start.

constexpr int kBWaves = 8;  // waves of a balanced-split workgroup (one per CU)
constexpr int kTileBufs = 2;  // K/V tile buffers per wave (tiles in flight + 1)
constexpr int kBThreads = kBWaves * kWave;

// Workgroups are dispatched to the GPU's 8 XCDs in turn (workgroup b to XCD
// b mod 8), and each XCD has its own L2.  Logical index of workgroup b of n
// that gives each XCD one contiguous range of indices, so that neighbouring
// shares (the samples of one prompt, next to each other in the sequence
// list, read the same prompt blocks at the same time) run behind one L2.
// A bijection of [0, n) for any n.
__device__ inline int xcd_contiguous(int b, int n) {
  constexpr int kXcds = 8;
  const int q = n / kXcds, r = n - q * kXcds;
  const int x = b % kXcds, i = b / kXcds;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Number of the worker whose share [j T / n, (j + 1) T / n) holds item u.
__device__ inline int worker_of(int64_t u, int64_t total, int32_t num_workers) {
  return (int)(((u + 1) * num_workers - 1) / total);
}

template <int D, int B, int G, bool kAppend>
__global__ __launch_bounds__(kBThreads) void decode_balanced_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    int32_t table_width, const int32_t* __restrict__ context_lens, uint16_t* __restrict__ out,
    int2* __restrict__ meta, float* __restrict__ part_ml, float* __restrict__ part_o,
    int32_t num_seqs, int32_t num_kv_heads, int32_t num_blocks, int32_t max_context_len,
    int32_t num_groups, int32_t gs, float qscale, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, uint16_t* k_dst, uint16_t* v_dst) {
  constexpr int DT = D / 16;
  extern __shared__ int32_t sm_dyn[];
  int32_t* sm_c = sm_dyn;                 // [num_seqs + 1] tiles of one chunk before sequence s
  int32_t* sm_n = sm_dyn + num_seqs + 1;  // [num_seqs] clamped context lengths
  __shared__ int32_t sm_scan[kBWaves];    // wave totals of the scan

  // Prefix sums of the tile counts (every workgroup computes its own copy).
  {
    const int per = (num_seqs + kBThreads - 1) / kBThreads;
    const int i0 = min(num_seqs, (int)threadIdx.x * per);
    const int i1 = min(num_seqs, i0 + per);
    int local = 0;
    for (int i = i0; i < i1; ++i) {
      // Lengths outside [0, max_context_len] break the caller's contract;
      // clamping keeps every access in bounds regardless.
      const int n = min(max(context_lens[i], 0), max_context_len);
      sm_n[i] = n;
      local += (n + kTile - 1) / kTile;
    }
    // Inclusive scan of `local`: within each wave by lane shuffles, then the
    // wave totals through LDS (one barrier instead of two per scan step).
    const int ln = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    int x = local;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off, kWave);
      if (ln >= off) x += y;
    }
    if (ln == kWave - 1) sm_scan[wv] = x;
    __syncthreads();
    int run = x - local;
    for (int v = 0; v < wv; ++v) run += sm_scan[v];
    for (int i = i0; i < i1; ++i) {
      sm_c[i] = run;
      run += (sm_n[i] + kTile - 1) / kTile;
    }
    // the last thread's running sum is the total (its own sequences included)
    if (threadIdx.x == kBThreads - 1) sm_c[num_seqs] = run;
    __syncthreads();
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int hq = num_kv_heads * G;
  // No worker covers an empty sequence: its outputs are zeros here, and its
  // pairs are marked so that the combine kernel skips them.
  for (int i = blockIdx.x; i < num_seqs; i += gridDim.x) {
    if (sm_n[i] != 0) continue;
    for (int e = threadIdx.x; e < hq * D; e += kBThreads) out[(int64_t)i * hq * D + e] = 0;
    for (int g = threadIdx.x; g < num_kv_heads; g += kBThreads)
      meta[(int64_t)i * num_kv_heads + g] = make_int2(-1, -1);
  }
  if constexpr (kAppend) {
    // The appended rows go to their slots here, before any worker starts, so
    // no store sits in the workers' pipelined loop; the workers read those
    // rows from k_new / v_new, never from the slots written here.
    constexpr int kChunks = D / 8;
    const int per_seq = 2 * num_kv_heads * kChunks;  // K and V, 16-byte pieces
    for (int i = blockIdx.x; i < num_seqs; i += gridDim.x) {
      const int t = sm_n[i] - 1;
      if (t < 0) continue;
      const int phys = block_tables[(int64_t)i * table_width + t / B];
      if (phys < 0 || phys >= num_blocks) continue;
      for (int e = threadIdx.x; e < per_seq; e += kBThreads) {
        const int which = e / (num_kv_heads * kChunks);
        const int r = e - which * num_kv_heads * kChunks;
        const int g = r / kChunks;
        const int c = r - g * kChunks;
        const int64_t src = ((int64_t)i * num_kv_heads + g) * D + 8 * c;
        const int64_t dst = (((int64_t)phys * num_kv_heads + g) * B + t % B) * D + 8 * c;
        const uint4 x = *reinterpret_cast<const uint4*>((which ? v_new : k_new) + src);
        *reinterpret_cast<uint4*>((which ? v_dst : k_dst) + dst) = x;
      }
    }
  }
  const int chunks = num_kv_heads / gs;
  const int64_t total = (int64_t)chunks * sm_c[num_seqs];
  // With fewer items than groups only the first `total` groups take one
  // each: every group in [0, ng) has a non-empty share, so the groups that
  // cover a sequence's chunk are exactly the range between its first and
  // last item's.
  const int ng = (int)min((int64_t)num_groups, total);
  // gs divides kBWaves: groups stay in a workgroup
  const int wg = xcd_contiguous(blockIdx.x, gridDim.x) * kBWaves + wave;
  const int j = wg / gs;                       // this wave's group (worker)
  const int hi = wg - j * gs;                  // its head within the chunk
  if (j >= ng) return;  // no barrier follows: the waves are independent from here
  const int64_t u0 = (int64_t)j * total / ng;
  const int64_t u1 = (int64_t)(j + 1) * total / ng;

  // An item's place: sequence, chunk, tile index in the chunk's pair, the
  // sequence's tile count and length (all wave-uniform).  This wave's head is
  // g = c gs + hi.
  struct Pos {
    int s, c, tile, nt, n;
  };
  auto seq_info = [&](Pos& x) {
    x.nt = __builtin_amdgcn_readfirstlane(sm_c[x.s + 1] - sm_c[x.s]);
    x.n = __builtin_amdgcn_readfirstlane(sm_n[x.s]);
  };
  auto pos_of = [&](int64_t u) {
    // The last sequence whose first item is <= u: the first items do not
    // decrease, so it is one less than the number of sequences starting at or
    // before u, counted 64 at a time with a ballot.
    int count = 0;
    for (int c = 0; c < num_seqs; c += kWave) {
      const int jj = c + lane;
      const bool at_or_before = jj < num_seqs && (int64_t)chunks * sm_c[jj] <= u;
      count += __builtin_popcountll(__builtin_amdgcn_ballot_w64(at_or_before));
    }
    Pos x;
    x.s = __builtin_amdgcn_readfirstlane(count - 1);
    seq_info(x);
    const int64_t r = u - (int64_t)chunks * __builtin_amdgcn_readfirstlane(sm_c[x.s]);
    x.c = (int)(r / x.nt);
    x.tile = (int)(r - (int64_t)x.c * x.nt);
    return x;
  };
  auto next = [&](Pos x) {  // only called for items before u1, so the result is an item
    if (++x.tile < x.nt) return x;
    x.tile = 0;
    if (++x.c < chunks) return x;
    x.c = 0;
    do {
      ++x.s;
    } while (__builtin_amdgcn_readfirstlane(sm_c[x.s + 1]) == __builtin_amdgcn_readfirstlane(sm_c[x.s]));
    seq_info(x);
    return x;
  };
  // The tile of the sequence processed at place x.tile.  The chunks of one
  // sequence start their tiles at different places (rotated by c nt /
  // chunks), so groups on different chunks of one sequence, which move
  // through it side by side, do not read the same physical blocks at the
  // same moment; the waves of one group do, on purpose.
  auto ptile = [&](const Pos& x) {
    const int r = x.tile + (x.c * x.nt) / chunks;
    return r >= x.nt ? r - x.nt : r;
  };
  // Block-table entry of this lane's row of tile x (a valid entry of the
  // sequence's row even for rows past its end).
  auto table_entry = [&](const Pos& x) {
    const int t = min(ptile(x) * kTile + col, x.n - 1);
    return block_tables[(int64_t)x.s * table_width + t / B];
  };
  const uint16_t* safe = q + 8 * grp;
  // With kAppend the row of position n - 1 (the token appended this step)
  // comes from k_new / v_new [num_seqs, Hkv, D] instead of the cache (the
  // prologue stored it into the cache slot: the same bits either way).
  auto load_tile = [&](const Pos& x, int phys, bool live, KVTile<D>& kv) {
    const int t = ptile(x) * kTile + col;
    const int g = x.c * gs + hi;
    const uint16_t* kr = nullptr;
    const uint16_t* vr = nullptr;
    if constexpr (kAppend) {
      const int64_t nrow = ((int64_t)x.s * num_kv_heads + g) * D + 8 * grp;
      kr = t == x.n - 1 ? k_new + nrow : nullptr;
      vr = t == x.n - 1 ? v_new + nrow : nullptr;
    }
    load_kv<D, B>(kv, k_cache, v_cache, safe, live && t < x.n, phys, t, g, num_kv_heads,
                  num_blocks, grp, kr, vr);
  };
  auto qrow = [&](const Pos& x) { return q + ((int64_t)x.s * hq + (x.c * gs + hi) * G) * D; };

  MfmaAttn<D, G> at;
  at.init(col, grp);
  int64_t seg_u0 = u0;  // first item of the current segment

  // Update with item u (place x); at the end of a segment write its result
  // and prepare for the next (sequence, chunk) (place nx).
  auto step = [&](const Pos& x, int64_t u, KVTile<D>& kv, const Pos& nx) {
    at.update(kv, min(kTile, x.n - ptile(x) * kTile), qscale, grp);
    if (x.tile + 1 < x.nt && u + 1 < u1) return;
    const int64_t pair_u0 = (int64_t)chunks * sm_c[x.s] + (int64_t)x.c * x.nt;
    const int g = x.c * gs + hi;
    const int pair = x.s * num_kv_heads + g;
    const bool first = seg_u0 == pair_u0;
    const bool whole = first && u + 1 == pair_u0 + x.nt;
    const float l = rows_sum(at.l);
    if (col < G) {
      const int64_t row = (int64_t)x.s * hq + g * G + col;
      if (whole) {
#pragma unroll
        for (int jj = 0; jj < DT; ++jj) {
          uint2 v;
          v.x = (uint32_t)f32_to_bf16_rne(at.o[jj][0] / l) |
                ((uint32_t)f32_to_bf16_rne(at.o[jj][1] / l) << 16);
          v.y = (uint32_t)f32_to_bf16_rne(at.o[jj][2] / l) |
                ((uint32_t)f32_to_bf16_rne(at.o[jj][3] / l) << 16);
          *reinterpret_cast<uint2*>(out + row * D + 16 * jj + 4 * grp) = v;
        }
      } else {
        const int64_t slot = (((int64_t)x.s * chunks + x.c + j) * gs + hi) * G + col;
#pragma unroll
        for (int jj = 0; jj < DT; ++jj)
          *reinterpret_cast<float4*>(part_o + slot * D + 16 * jj + 4 * grp) =
              make_float4(at.o[jj][0], at.o[jj][1], at.o[jj][2], at.o[jj][3]);
        if (grp == 0) *reinterpret_cast<float2*>(part_ml + slot * 2) = make_float2(at.m, l);
      }
    }
    if (first && lane == 0)
      meta[pair] = make_int2(j, worker_of(pair_u0 + x.nt - 1, total, ng));
    if (u + 1 < u1) {
      at.reset();
      at.load_q(qrow(nx), col, grp);
      seg_u0 = u + 1;
    }
  };

  // Pipeline over kTileBufs tile buffers: while item u is processed, the K/V
  // of items u + 1 .. u + kTileBufs - 1 and the table entry of the item after
  // them are in flight.  The item count is padded to a multiple of kTileBufs
  // (dummy items load a safe row and are not processed) so the loop has one
  // exit and the compiler's load counting stays exact across the back edge.
  // p[f] holds the place of item u + f at the top of each round; each step
  // replaces its own place with that of the item kTileBufs later.
  constexpr int NBF = kTileBufs;
  Pos p[NBF];
  KVTile<D> t[NBF];
  p[0] = pos_of(u0);
  at.load_q(qrow(p[0]), col, grp);
#pragma unroll
  for (int f = 1; f < NBF; ++f) p[f] = u0 + f < u1 ? next(p[f - 1]) : p[f - 1];
#pragma unroll
  for (int f = 0; f < NBF - 1; ++f) load_tile(p[f], table_entry(p[f]), u0 + f < u1, t[f]);
  int ph = table_entry(p[NBF - 1]);  // entry of the next item to load
  for (int64_t u = u0; u < u1; u += NBF) {
#pragma unroll
    for (int f = 0; f < NBF; ++f) {
      const int lb = (f + NBF - 1) % NBF;  // buffer (and place) of item u + f + NBF - 1
      load_tile(p[lb], ph, u + f + NBF - 1 < u1, t[lb]);
      const Pos pn = u + f + NBF < u1 ? next(p[lb]) : p[lb];
      ph = table_entry(pn);
      if (u + f < u1) step(p[f], u + f, t[f], p[(f + 1) % NBF]);
      p[f] = pn;
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

// One wave per (pair, query head) of the balanced split: pairs covered by
// several workers are combined here, in worker order,
// out = sum_w o_w 2^(m_w - m*) / sum_w L_w 2^(m_w - m*).  Pairs finished by a
// single worker, and pairs of empty sequences, are left alone.  Contributors
// are taken 64 at a time: lane j fetches contributor j's (m, L) while every
// lane fetches its D / 64 output dims of the group's first kFirst
// contributors; the group's maximum and weighted sum come from wave
// reductions, then each lane folds its dims, so a pair split over up to
// kFirst workers costs one round trip after the record of its workers (the
// output dims of further contributors follow kChunk at a time).  Four such waves share a
// workgroup: dispatching one-wave workgroups costs about as much as the whole
// combine.
template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_balanced_reduce_kernel(
    uint16_t* __restrict__ out, const int2* __restrict__ meta, const float* __restrict__ part_ml,
    const float* __restrict__ part_o, int32_t num_pairs, int32_t num_kv_heads, int32_t num_workers,
    int32_t gs) {
  constexpr int DPL = D / kWave;  // dims per lane
  constexpr int kFirst = 8;       // contributors fetched with the (m, L) of their group
  constexpr int kChunk = 32;      // contributors fetched per later round
  static_assert(DPL * kWave == D, "head_dim must be a multiple of 64");
  const int unit = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (unit >= num_pairs * G) return;
  const int pair = unit / G;
  const int h = unit - pair * G;
  const int lane = threadIdx.x & (kWave - 1);
  const int2 mt = meta[pair];
  const int wa = max(mt.x, 0), wb = min(mt.y, num_workers - 1);
  if (mt.x < 0 || wa >= wb) return;
  const int nseg = wb - wa + 1;
  // The pair (sequence s, KV head g) is item chunk pc = s chunks + g / gs of
  // the work list; worker k wrote its partial to slot (pc + k) gs + g % gs.
  const int s = pair / num_kv_heads;
  const int g = pair - s * num_kv_heads;
  const int64_t pc = (int64_t)s * (num_kv_heads / gs) + g / gs;
  const int64_t slot0 = (pc + wa) * gs + g % gs;
  const int64_t stride = (int64_t)gs * G;  // rows between consecutive workers' slots
  const float* ml = part_ml + (slot0 * G + h) * 2;  // worker wa + k at ml[k * 2 stride]
  const float* po = part_o + (slot0 * G + h) * D + lane * DPL;
  float M = -INFINITY, L = 0.0f, O[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) O[e] = 0.0f;
  for (int k0 = 0; k0 < nseg; k0 += kWave) {
    const int ng = min(kWave, nseg - k0);  // contributors in this group
    const bool mine = lane < ng;
    // Unpredicated loads with clamped indices (a lane past the group re-reads
    // the last contributor and its factor is zero), the first kFirst
    // contributors' output dims issued with the (m, L) loads in one block,
    // before any of them is waited for.
    float2 v = *reinterpret_cast<const float2*>(ml + (int64_t)(k0 + min(lane, ng - 1)) * 2 * stride);
    auto fetch = [&](auto& ov, int c0) {
      constexpr int kc = sizeof(ov) / sizeof(ov[0]);
#pragma unroll
      for (int c = 0; c < kc; ++c) {
        const int64_t k = k0 + min(c0 + c, ng - 1);
#pragma unroll
        for (int e = 0; e < DPL; ++e) ov[c][e] = po[k * stride * D + e];
      }
    };
    float ov0[kFirst][DPL];
    fetch(ov0, 0);
    if (!mine) v = make_float2(-INFINITY, 0.0f);
    const float cm = fmaxf(M, group_max<kWave>(v.x));
    const float a = M == -INFINITY ? 0.0f : exp2f(M - cm);  // rescales what came before
    const float f = mine ? exp2f(v.x - cm) : 0.0f;          // lane j: contributor k0 + j's factor
    L = fmaf(L, a, group_sum<kWave>(v.y * f));
#pragma unroll
    for (int e = 0; e < DPL; ++e) O[e] *= a;
    auto add = [&](const auto& ov, int c0) {
      constexpr int kc = sizeof(ov) / sizeof(ov[0]);
#pragma unroll
      for (int c = 0; c < kc; ++c) {
        // contributors past the group are selected out, not multiplied by 0
        const float fc = __int_as_float(
            __builtin_amdgcn_readlane(__float_as_int(f), min(c0 + c, kWave - 1)));
#pragma unroll
        for (int e = 0; e < DPL; ++e) O[e] = c0 + c < ng ? fmaf(ov[c][e], fc, O[e]) : O[e];
      }
    };
    add(ov0, 0);
    for (int c0 = kFirst; c0 < ng; c0 += kChunk) {
      float ov[kChunk][DPL];
      fetch(ov, c0);
      add(ov, c0);
    }
    M = cm;
  }
  uint16_t* orow = out + ((int64_t)pair * G + h) * D + lane * DPL;
#pragma unroll
  for (int e = 0; e < DPL; ++e) store_out(orow + e, O[e] / L);
}

// ------------------------------------------------------------- dispatch

constexpr int kWorkerWavesPerSimd = 2;  // the balanced kernel's occupancy (VGPR-bound)
// Static LDS of the balanced kernel (the wave totals of its scan, sm_scan);
// the dynamic part is (2 num_seqs + 1) int32 of prefix sums and lengths.
constexpr int kBalancedStaticLds = kBWaves * (int)sizeof(int32_t);
// Balanced-split workgroups resident on one CU (kBWaves waves each).
constexpr int kBalancedWgPerCu = 4 * kWorkerWavesPerSimd / kBWaves;
static_assert(kBalancedWgPerCu >= 1, "a balanced workgroup must fit one CU");

// Waves of one balanced-split worker group: the largest power of two up to
// kBWaves that divides the KV head count (the group's waves take that many
// heads of one sequence).
int32_t group_size(int32_t num_kv_heads) {
  int32_t gs = kBWaves;
  while (num_kv_heads % gs) gs /= 2;
  return gs;
}

// How one call is split and where its workspace pieces go.
struct Plan {
  bool balanced;
  int32_t parts;    // split-context: partitions per sequence
  int32_t ps;       // split-context: tokens per partition
  int32_t workers;  // balanced: waves
  int32_t gs;       // balanced: waves per worker group
  size_t meta_off, ml_off, o_off, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// What the balanced split needs to know about the current device: its
// workers (the waves it holds at once: CUs x 4 SIMDs x kWorkerWavesPerSimd)
// and the most sequences whose prefix sums and lengths fit the LDS one of its
// workgroups may use.  The grid puts kBalancedWgPerCu workgroups on every CU,
// so a workgroup may use that share of the CU's LDS (and no more than the
// per-workgroup maximum).
struct DeviceLimits {
  int32_t workers;
  int32_t max_seqs;
};

int device_limits(DeviceLimits* out) {
  static std::mutex mu;
  static DeviceLimits cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pkv__fail(PKV_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 0 && dev < 64 && cache[dev].workers > 0) {
    *out = cache[dev];
    return PKV_OK;
  }
  int cus = 0, lds_cu = 0, lds_block = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&lds_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess || cus <= 0 || lds_cu <= 0 || lds_block <= 0)
    return pkv__fail(PKV_EHIP, "device attributes: %s", hipGetErrorString(e));
  const int budget = std::min(lds_block, lds_cu / kBalancedWgPerCu);
  DeviceLimits d;
  d.workers = cus * 4 * kWorkerWavesPerSimd;
  d.max_seqs = std::max(0, (budget - kBalancedStaticLds - (int)sizeof(int32_t)) /
                               (2 * (int)sizeof(int32_t)));
  if (dev >= 0 && dev < 64) cache[dev] = d;
  *out = d;
  return PKV_OK;
}

int make_plan(const pkv_cache_desc* c, int32_t num_seqs, int32_t num_q_heads,
              int32_t max_context_len, int32_t partition_size, Plan* pl) {
  const int32_t B = c->block_size, D = c->head_dim;
  const int32_t G = num_q_heads / c->num_kv_heads;
  *pl = Plan{};
  if (partition_size == PKV_PARTITION_AUTO) {
    const int64_t tiles_per_head = (int64_t)num_seqs * ((max_context_len + kTile - 1) / kTile);
    DeviceLimits lim{0, 0};
    if (c->dtype == PKV_BF16) {
      int rc = device_limits(&lim);
      if (rc) return rc;
    }
    if (c->dtype == PKV_BF16 && num_seqs <= lim.max_seqs && tiles_per_head < (1 << 30)) {
      const int32_t nw = lim.workers;
      const size_t pairs = (size_t)num_seqs * c->num_kv_heads;
      const size_t slots = (pairs + (size_t)nw) * G;
      pl->balanced = true;
      pl->workers = nw;
      pl->gs = group_size(c->num_kv_heads);
      pl->meta_off = 0;
      pl->ml_off = align256(pairs * sizeof(int2));
      pl->o_off = pl->ml_off + align256(slots * 2 * sizeof(float));
      pl->bytes = pl->o_off + slots * (size_t)D * sizeof(float);
      return PKV_OK;
    }
    partition_size = 512;  // a multiple of every compiled block size
  }
  const int32_t parts = (partition_size <= 0 || max_context_len <= 0)
                            ? 1
                            : (max_context_len + partition_size - 1) / partition_size;
  pl->parts = parts;
  // With no split, one partition holds the longest context.
  pl->ps = parts == 1 ? (max_context_len > 0 ? ((max_context_len + B - 1) / B) * B : B)
                      : partition_size;
  if (parts > 1) {
    const size_t rows = (size_t)num_seqs * num_q_heads * parts;
    pl->ml_off = 0;
    pl->o_off = rows * 2 * sizeof(float);
    pl->bytes = pl->o_off + rows * (size_t)D * sizeof(float);
  }
  return PKV_OK;
}

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
  const void* k_new;  // non-null: fused append (balanced split only)
  const void* v_new;
  Plan plan;
  float qscale;
  int2* meta;
  float* part_ml;
  float* part_o;
  hipStream_t stream;
  hipEvent_t mark_before;  // non-null: recorded around the first kernel
  hipEvent_t mark_after;
};

// Events the next decode call on this thread records around its first
// kernel (pkv_decode_mark_next_call); each call takes them and clears them.
thread_local hipEvent_t t_mark_before = nullptr;
thread_local hipEvent_t t_mark_after = nullptr;

// Launch `kernel`; with marks, through hipExtLaunchKernel, whose start and
// stop events the dispatch itself records as the kernel starts and ends.
template <typename... KArgs, typename... Args>
void launch_marked(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds, hipStream_t st,
                   hipEvent_t before, hipEvent_t after, Args... args) {
  if (before)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, before, after, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv__fail(PKV_EHIP, "%s launch: %s", what, hipGetErrorString(e));
  return PKV_OK;
}

template <typename E, int D, int B, int G>
int launch(const LaunchArgs& a) {
  if constexpr (E::bytes == 2) {
    if (a.plan.balanced) {
      const size_t lds = (size_t)(2 * a.num_seqs + 1) * sizeof(int32_t);
      const int32_t groups = a.plan.workers / a.plan.gs;
      const dim3 grid((uint32_t)(a.plan.workers / kBWaves));
      if (a.k_new)
        launch_marked(decode_balanced_kernel<D, B, G, true>, grid, dim3(kBThreads),
                      (uint32_t)lds, a.stream, a.mark_before, a.mark_after,
                      (const uint16_t*)a.q, (const uint16_t*)a.k_cache,
                      (const uint16_t*)a.v_cache, a.block_tables, a.width, a.context_lens,
                      (uint16_t*)a.out, a.meta, a.part_ml, a.part_o, a.num_seqs, a.num_kv_heads,
                      a.num_blocks, a.max_context_len, groups, a.plan.gs, a.qscale,
                      (const uint16_t*)a.k_new, (const uint16_t*)a.v_new, (uint16_t*)a.k_cache,
                      (uint16_t*)a.v_cache);
      else
        launch_marked(decode_balanced_kernel<D, B, G, false>, grid, dim3(kBThreads),
                      (uint32_t)lds, a.stream, a.mark_before, a.mark_after,
                      (const uint16_t*)a.q, (const uint16_t*)a.k_cache,
                      (const uint16_t*)a.v_cache, a.block_tables, a.width, a.context_lens,
                      (uint16_t*)a.out, a.meta, a.part_ml, a.part_o, a.num_seqs, a.num_kv_heads,
                      a.num_blocks, a.max_context_len, groups, a.plan.gs, a.qscale,
                      (const uint16_t*)nullptr, (const uint16_t*)nullptr, (uint16_t*)nullptr,
                      (uint16_t*)nullptr);
      int rc = check_launch("decode_balanced");
      if (rc) return rc;
      const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * G;
      hipLaunchKernelGGL((decode_balanced_reduce_kernel<D, G>),
                         dim3((uint32_t)((units + kWaves - 1) / kWaves)), dim3(kThreads), 0,
                         a.stream, (uint16_t*)a.out, (const int2*)a.meta, (const float*)a.part_ml,
                         (const float*)a.part_o, a.num_seqs * a.num_kv_heads, a.num_kv_heads,
                         groups, a.plan.gs);
      return check_launch("decode_balanced_reduce");
    }
  }
  const int64_t grid = (int64_t)a.num_seqs * a.num_kv_heads * a.plan.parts;
  if (grid > INT32_MAX) return pkv__fail(PKV_EINVAL, "decode grid too large");
  if constexpr (E::bytes == 2) {
    launch_marked(decode_partition_mfma_kernel<D, B, G>, dim3((uint32_t)grid), dim3(kThreads), 0u,
                  a.stream, a.mark_before, a.mark_after, (const uint16_t*)a.q,
                  (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.block_tables, a.width,
                  a.context_lens, (uint16_t*)a.out, a.part_ml, a.part_o, a.num_seqs,
                  a.num_kv_heads, a.num_blocks, a.plan.parts, a.plan.ps, a.max_context_len,
                  a.qscale);
  } else {
    launch_marked(decode_partition_valu_kernel<E, D, B, G>, dim3((uint32_t)grid), dim3(kThreads),
                  0u, a.stream, a.mark_before, a.mark_after, (const typename E::raw*)a.q,
                  (const uint4*)a.k_cache, (const uint4*)a.v_cache, a.block_tables, a.width,
                  a.context_lens, (typename E::raw*)a.out, a.part_ml, a.part_o, a.num_seqs,
                  a.num_kv_heads, a.num_blocks, a.plan.parts, a.plan.ps, a.max_context_len,
                  a.qscale);
  }
  int rc = check_launch("decode_partition");
  if (rc) return rc;
  if (a.plan.parts > 1) {
    hipLaunchKernelGGL((decode_reduce_kernel<E, D>), dim3((uint32_t)(a.num_seqs * a.num_q_heads)),
                       dim3(D), 0, a.stream, (typename E::raw*)a.out, a.part_ml, a.part_o,
                       a.context_lens, a.num_q_heads, a.plan.parts, a.plan.ps, a.max_context_len);
    return check_launch("decode_reduce");
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

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_sizes(const pkv_cache_desc* c, int32_t num_seqs, int32_t num_q_heads,
                int32_t max_context_len, int32_t partition_size) {
  int rc = pkv__check_desc(c);
  if (rc) return rc;
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0)
    return pkv__fail(PKV_EINVAL, "bad sizes (num_seqs=%d num_q_heads=%d max_context_len=%d)",
                     num_seqs, num_q_heads, max_context_len);
  if (num_q_heads % c->num_kv_heads != 0)
    return pkv__fail(PKV_EINVAL, "num_q_heads %d is not a multiple of num_kv_heads %d",
                     num_q_heads, c->num_kv_heads);
  if (partition_size != PKV_PARTITION_AUTO &&
      (partition_size < 0 || (partition_size > 0 && partition_size % c->block_size != 0)))
    return pkv__fail(PKV_EINVAL,
                     "partition_size %d must be PKV_PARTITION_AUTO, 0 or a positive multiple of "
                     "block_size %d", partition_size, c->block_size);
  return PKV_OK;
}

}  // namespace

extern "C" size_t pkv_decode_workspace_bytes(const pkv_cache_desc* c, int32_t num_seqs,
                                             int32_t num_q_heads, int32_t max_context_len,
                                             int32_t partition_size) {
  pkv__clear_error();
  if (check_sizes(c, num_seqs, num_q_heads, max_context_len, partition_size) || num_seqs == 0)
    return 0;
  Plan pl;
  if (make_plan(c, num_seqs, num_q_heads, max_context_len, partition_size, &pl)) return 0;
  return pl.bytes;
}

extern "C" int pkv_decode_mark_next_call(void* before, void* after) {
  pkv__clear_error();
  if ((before == nullptr) != (after == nullptr))
    return pkv__fail(PKV_EINVAL, "give both events or neither");
  t_mark_before = (hipEvent_t)before;
  t_mark_after = (hipEvent_t)after;
  return PKV_OK;
}

extern "C" int32_t pkv_decode_balanced_max_seqs(void) {
  pkv__clear_error();
  DeviceLimits lim;
  if (device_limits(&lim)) return -1;
  return lim.max_seqs;
}

namespace {

int decode_impl(void* out, const void* q, const void* k_new, const void* v_new,
                const void* k_cache, const void* v_cache, const pkv_cache_desc* c,
                const int32_t* block_tables, int32_t max_blocks_per_seq,
                const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                int32_t max_context_len, float scale, int32_t partition_size, void* workspace,
                size_t workspace_bytes, void* stream) {
  // the marks belong to this call, whatever it returns
  const hipEvent_t mark_before = t_mark_before, mark_after = t_mark_after;
  t_mark_before = t_mark_after = nullptr;
  int rc = check_sizes(c, num_seqs, num_q_heads, max_context_len, partition_size);
  if (rc) return rc;
  if (max_blocks_per_seq < 0 || (int64_t)max_blocks_per_seq * c->block_size < max_context_len)
    return pkv__fail(PKV_EINVAL, "table width %d * block_size %d < max_context_len %d",
                     max_blocks_per_seq, c->block_size, max_context_len);
  if (!(scale == scale) || isinf(scale)) return pkv__fail(PKV_EINVAL, "scale is not finite");
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return pkv__fail(PKV_EINVAL, "NULL device pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      ((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u))
    return pkv__fail(PKV_EINVAL, "q, out and caches must be 16-byte aligned");

  Plan pl;
  rc = make_plan(c, num_seqs, num_q_heads, max_context_len, partition_size, &pl);
  if (rc) return rc;
  if (k_new) {
    if (!v_new) return pkv__fail(PKV_EINVAL, "v_new is NULL");
    if (!pl.balanced)
      return pkv__fail(PKV_EUNSUPPORTED,
                       "the fused append runs in the balanced split only (bf16 caches, "
                       "PKV_PARTITION_AUTO, num_seqs <= pkv_decode_balanced_max_seqs())");
    if (!aligned16(k_new) || !aligned16(v_new))
      return pkv__fail(PKV_EINVAL, "k_new and v_new must be 16-byte aligned");
  }
  if (workspace_bytes < pl.bytes || (pl.bytes && !workspace))
    return pkv__fail(PKV_EINVAL, "workspace of %zu bytes is smaller than the %zu needed",
                     workspace_bytes, pl.bytes);
  if (pl.bytes && !aligned16(workspace))
    return pkv__fail(PKV_EINVAL, "workspace must be 16-byte aligned");

  if (pkv__validate_enabled()) {
    // debug: the contract of tables and lengths, checked on the host first
    const size_t nt = (size_t)num_seqs * max_blocks_per_seq;
    int32_t* ht = (int32_t*)malloc((nt ? nt : 1) * sizeof(int32_t));
    int32_t* hc = (int32_t*)malloc((size_t)num_seqs * sizeof(int32_t));
    rc = (ht && hc) ? PKV_OK : pkv__fail(PKV_EINVAL, "out of host memory");
    if (!rc && nt) rc = pkv__copy_to_host(ht, block_tables, nt * sizeof(int32_t), stream);
    if (!rc) rc = pkv__copy_to_host(hc, context_lens, (size_t)num_seqs * sizeof(int32_t), stream);
    if (!rc)
      rc = pkv_validate_decode(ht, max_blocks_per_seq, hc, num_seqs, max_context_len, c);
    free(ht);
    free(hc);
    if (rc) return rc;
  }

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
  a.k_new = k_new;
  a.v_new = v_new;
  a.plan = pl;
  a.qscale = scale * kLog2e;
  char* ws = (char*)workspace;
  a.meta = pl.bytes ? (int2*)(ws + pl.meta_off) : nullptr;
  a.part_ml = pl.bytes ? (float*)(ws + pl.ml_off) : nullptr;
  a.part_o = pl.bytes ? (float*)(ws + pl.o_off) : nullptr;
  a.stream = (hipStream_t)stream;
  a.mark_before = mark_before;
  a.mark_after = mark_after;
  const int G = num_q_heads / c->num_kv_heads;
  if (c->dtype == PKV_BF16) return dispatch_d<BF16>(a, c->head_dim, c->block_size, G);
  return dispatch_d<F32>(a, c->head_dim, c->block_size, G);
}

}  // namespace

extern "C" int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                                          const void* v_cache, const pkv_cache_desc* c,
                                          const int32_t* block_tables,
                                          int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_q_heads, int32_t max_context_len,
                                          float scale, int32_t partition_size, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  pkv__clear_error();
  return decode_impl(out, q, nullptr, nullptr, k_cache, v_cache, c, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, num_q_heads, max_context_len,
                     scale, partition_size, workspace, workspace_bytes, stream);
}

// ------------------------------------------------- allocation-free variant
//
// pkv_paged_attention_decode_noalloc keeps its workspace (the balanced split's
// worker records and partials, or the split-context partials) in this
// file-scope device array instead of a caller-supplied buffer.  Every device
// the library runs on holds its own copy until the process ends.  On the host
// `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kScratchBytes = PKV_DECODE_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device (looked up on the first
// call made with that device current).
int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pkv__fail(PKV_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pkv__fail(PKV_EUNSUPPORTED, "device %d: the scratch table holds %d devices", dev,
                     kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return pkv__fail(PKV_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_paged_attention_decode_noalloc(
    void* out, const void* q, const void* k_cache, const void* v_cache, const pkv_cache_desc* c,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len, float scale,
    int32_t partition_size, void* stream) {
  pkv__clear_error();
  int rc = check_sizes(c, num_seqs, num_q_heads, max_context_len, partition_size);
  if (rc || num_seqs == 0) t_mark_before = t_mark_after = nullptr;  // no launch follows
  if (rc) return rc;
  if (num_seqs == 0) return PKV_OK;
  Plan pl;
  rc = make_plan(c, num_seqs, num_q_heads, max_context_len, partition_size, &pl);
  if (rc || pl.bytes > kScratchBytes) t_mark_before = t_mark_after = nullptr;
  if (rc) return rc;
  if (pl.bytes > kScratchBytes)
    return pkv__fail(PKV_EINVAL,
                     "this decode needs %zu bytes of workspace, more than the %zu bytes of "
                     "library scratch; call pkv_paged_attention_decode with a workspace",
                     pl.bytes, kScratchBytes);
  void* ws = nullptr;
  if (pl.bytes) {
    rc = scratch_address(&ws);
    if (rc) {
      t_mark_before = t_mark_after = nullptr;
      return rc;
    }
  }
  return decode_impl(out, q, nullptr, nullptr, k_cache, v_cache, c, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, num_q_heads, max_context_len,
                     scale, partition_size, ws, ws ? kScratchBytes : 0, stream);
}

extern "C" int pkv_paged_attention_decode_append(
    void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    const pkv_cache_desc* c, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
    float scale, void* workspace, size_t workspace_bytes, void* stream) {
  pkv__clear_error();
  if (!k_new || !v_new) return pkv__fail(PKV_EINVAL, "NULL k_new or v_new");
  return decode_impl(out, q, k_new, v_new, k_cache, v_cache, c, block_tables, max_blocks_per_seq,
                     context_lens, num_seqs, num_q_heads, max_context_len, scale,
                     PKV_PARTITION_AUTO, workspace, workspace_bytes, stream);
}
