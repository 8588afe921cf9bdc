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

// D = A B + C on a 16x16x32 bf16 tile.  Lane l supplies row (l % 16) of A and
// column (l % 16) of B, each as 8 consecutive k-slots of group l / 16; it
// receives D[4 (l / 16) + r][l % 16] in element r.  Only the pairing of A's
// and B's k-slots matters to the kernel, not their order.
__device__ inline f32x4_t mfma16x16x32(const uint4& a, const uint4& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Two fp32 values that are exactly bf16 numbers -> one packed bf16 pair.
__device__ inline uint32_t pack_bf16_pair(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A tile's maximum must exceed the reference maximum by more than this (log2
// units) before the accumulators are rescaled; weights stay <= 2^8.
constexpr float kRescaleSlack = 8.0f;

template <int D, int B, int G>
__global__ __launch_bounds__(kThreads) void decode_partition_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    int32_t table_width, const int32_t* __restrict__ context_lens, uint16_t* __restrict__ out,
    float* __restrict__ part_ml, float* __restrict__ part_o, int32_t num_seqs,
    int32_t num_kv_heads, int32_t num_blocks, int32_t num_parts, int32_t ps,
    int32_t max_context_len, float qscale) {
  constexpr int KP = D / 32;           // 32-dim pieces of a row: one 16-byte load per lane each
  constexpr int DT = D / 16;           // 16-dim output tiles
  constexpr int kTile = 16;            // tokens per MFMA tile
  constexpr int kChunkTiles = 64;      // tiles whose table entries are staged at once
  constexpr int kChunkEntries = kChunkTiles * kTile / B + 2;
  static_assert(D % 32 == 0 && G >= 1 && G <= 16, "unsupported shape");

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

  // k-slot (grp, e) of piece kk is dim 32 kk + 8 grp + e, for K rows and q alike.
  uint4 qb[KP];
#pragma unroll
  for (int kk = 0; kk < KP; ++kk)
    qb[kk] = col < G ? *reinterpret_cast<const uint4*>(q + ((int64_t)s * hq + g * G + col) * D +
                                                       32 * kk + 8 * grp)
                     : make_uint4(0, 0, 0, 0);

  // Selection matrices: column c of half h picks dim 16 h + c of a 32-dim
  // piece, i.e. k-slot (2 h + c / 8, c % 8).  bf16 1.0 = 0x3f80.
  uint4 sel[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bool on = grp == 2 * h + (col >> 3);
    const int e = col & 7;
    const uint32_t one = 0x3f80u << (16 * (e & 1));
    sel[h] = make_uint4(on && (e >> 1) == 0 ? one : 0u, on && (e >> 1) == 1 ? one : 0u,
                        on && (e >> 1) == 2 ? one : 0u, on && (e >> 1) == 3 ? one : 0u);
  }

  f32x4_t o[DT];
#pragma unroll
  for (int j = 0; j < DT; ++j) o[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY;  // reference maximum of head `col` (log2 units)
  float l = 0.0f;       // this lane's share of the weight sum of head `col`

  __shared__ int32_t sm_bt[kChunkEntries];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  __shared__ float sm_o[kWaves][G][D];

  const int32_t* bt = block_tables + (int64_t)s * table_width;
  const int64_t blk_stride = (int64_t)num_kv_heads * B * D;
  const int64_t head_off = (int64_t)g * B * D + 8 * grp;

  // The K and V pieces of token row `col` of a tile.  The loads are not
  // predicated, so the compiler can keep the next tile's loads in flight
  // while the current tile is processed: a row past the partition (or whose
  // block id is outside the pool) reads this lane's query piece instead, a
  // small in-bounds row, and its V is replaced by zeros when it is used.
  const uint16_t* q_safe = q + ((int64_t)s * hq + g * G) * D + 8 * grp;
  struct Tile {
    uint4 k[KP], v[KP];
    bool ok;
  };
  auto load_tile = [&](int tile, int cb0, Tile& x) {
    const int t = t0 + tile * kTile + col;
    const bool live = tile >= 0 && t < t1;
    const int tc = live ? t : t1 - 1;  // stays inside the staged chunk
    const int phys = sm_bt[tc / B - cb0];
    x.ok = live && phys >= 0 && phys < num_blocks;
    const int64_t off = (int64_t)phys * blk_stride + head_off + (int64_t)(tc % B) * D;
    const uint16_t* kp = x.ok ? k_cache + off : q_safe;
    const uint16_t* vp = x.ok ? v_cache + off : q_safe;
#pragma unroll
    for (int kk = 0; kk < KP; ++kk) {
      x.k[kk] = *reinterpret_cast<const uint4*>(kp + 32 * kk);
      x.v[kk] = *reinterpret_cast<const uint4*>(vp + 32 * kk);
    }
  };

  auto process = [&](int tile, Tile& x) {
    // scores of tokens 4 grp + r (tile rows) for head `col`; rows that are
    // not live are replaced by -inf below, whatever their K bits were
    f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KP; ++kk) sc = mfma16x16x32(x.k[kk], qb[kk], sc);
    // V rows that are not live become zeros (their weight is 0, and 0 * NaN
    // would otherwise poison the output)
#pragma unroll
    for (int kk = 0; kk < KP; ++kk)
      if (!x.ok) x.v[kk] = make_uint4(0, 0, 0, 0);
    const int tb = t0 + tile * kTile + 4 * grp;
    float sv[4];
    float bm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = tb + r < t1 ? sc[r] * qscale : -INFINITY;
      bm = fmaxf(bm, sv[r]);
    }
    bm = fmaxf(bm, xor16(bm));
    bm = fmaxf(bm, xor32(bm));  // maximum over the tile's 16 tokens
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
#pragma unroll
    for (int j = 0; j < DT; ++j) {
      // V^T tile j: element r = V[token 4 grp + r][dim 16 j + col], exact
      const f32x4_t tv = mfma16x16x32(x.v[j >> 1], sel[j & 1], f32x4_t{0.0f, 0.0f, 0.0f, 0.0f});
      const uint32_t a01 = pack_bf16_pair(tv[0], tv[1]);
      const uint32_t a23 = pack_bf16_pair(tv[2], tv[3]);
      // o[j] element r += sum_t V[t][dim 16 j + 4 grp + r] * P[t][head col]
      o[j] = mfma16x16x32(make_uint4(a01, a23, a01, a23), pb, o[j]);
    }
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
    // Two tile buffers in turn: the loads of the tile after the current one
    // (or of a dummy row past the chunk's end) are issued before the current
    // tile is processed.
    Tile ta, tb;
    load_tile(tile, cb0, ta);
    for (;;) {
      load_tile(tile + kWaves < c1 ? tile + kWaves : -1, cb0, tb);
      process(tile, ta);
      tile += kWaves;
      if (tile >= c1) break;
      load_tile(tile + kWaves < c1 ? tile + kWaves : -1, cb0, ta);
      process(tile, tb);
      tile += kWaves;
      if (tile >= c1) break;
    }
  }

  // the four row groups of a head hold disjoint tokens' weight sums
  l += xor16(l);
  l += xor32(l);
  if (grp == 0 && col < G) {
    sm_m[wave][col] = m;
    sm_l[wave][col] = l;
  }
  if (col < G) {
#pragma unroll
    for (int j = 0; j < DT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm_o[wave][col][16 * j + 4 * grp + r] = o[j][r];
  }
  __syncthreads();
  merge_waves<uint16_t, D, G>(sm_m, sm_l, sm_o, (int64_t)s * hq + g * G, p, num_parts, nparts_s,
                              out, part_ml, part_o);
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
  if constexpr (E::bytes == 2) {
    hipLaunchKernelGGL((decode_partition_mfma_kernel<D, B, G>), dim3((uint32_t)grid),
                       dim3(kThreads), 0, a.stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.block_tables,
                       a.width, a.context_lens, (uint16_t*)a.out, a.part_ml, a.part_o,
                       a.num_seqs, a.num_kv_heads, a.num_blocks, a.num_parts, a.ps, a.max_context_len,
                       a.qscale);
  } else {
    hipLaunchKernelGGL((decode_partition_valu_kernel<E, D, B, G>), dim3((uint32_t)grid),
                       dim3(kThreads), 0, a.stream, (const typename E::raw*)a.q,
                       (const uint4*)a.k_cache, (const uint4*)a.v_cache, a.block_tables,
                       a.width, a.context_lens, (typename E::raw*)a.out, a.part_ml, a.part_o,
                       a.num_seqs, a.num_kv_heads, a.num_blocks, a.num_parts, a.ps, a.max_context_len,
                       a.qscale);
  }
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
