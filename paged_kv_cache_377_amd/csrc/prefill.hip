// Causal paged prefill attention for gfx950: several new tokens per sequence
// attend to their whole context through the block table, on MFMA (bf16 in,
// fp32 accumulation, bf16 out).
//
// What is computed (PagedAttention blog, 0539edu.com, section 3(3), step 1:
// the prompt's tokens are processed together and their K/V are filled into
// the sequence's blocks; read as causal attention over the prompt): sequence
// s owns query rows query_start_loc[s] .. query_start_loc[s + 1] - 1, its
// n_new new tokens, which are the last n_new of its context_lens[s] tokens
// (their K/V are written before this call, as for decode).  New token j sits
// at position p = context_lens[s] - n_new + j and attends to every position
// t <= p, keys and values read from block block_tables[s][t / B], offset
// t % B.  Query head h reads KV head h / G.
//
// Work decomposition.  A workgroup (4 waves) owns one KV head g of one
// sequence and 128 (token, head) rows: 128 / G consecutive new tokens times
// the G query heads that share g, token-major.  Each wave owns 32 rows as two
// 16-column MFMA tiles.  Keys are walked in tiles of 32 from position 0 to
// the tile's last position; each K/V tile is copied from HBM into LDS once
// per workgroup (rows in natural [key][dim] order) and read by all 4 waves,
// double-buffered so the next tile's loads are in flight during the MFMAs.
//
// Per key tile and wave:
//   S^T = K Q^T    (A = 16 keys x 32 dims of K from LDS, B = 32 dims x 16
//                   rows of Q held in registers): 2 key halves x D/32 steps
//                   x 2 column tiles of v_mfma_f32_16x16x32_bf16;
//   online softmax per row (a row is an MFMA column: lanes with equal l % 16
//                   hold its 8 keys of the tile), base-2 exponent, causal
//                   mask by position, lazy rescale;
//   O^T += V^T P^T (A = 16 dims x 32 keys of V^T, B = 32 keys x 16 rows of
//                   P): D/16 steps x 2 column tiles x 2 parts of P.  The B
//                   operand is the lane's own 8 probabilities in the order
//                   the S^T tiles left them; the A operand takes V in the
//                   same key order with the LDS transpose read
//                   (ds_read_b64_tr_b16), two per step.
// The probabilities enter the PV product as two bf16 parts, hi = bf16(p)
// and lo = bf16(p - hi) (round to nearest even), one MFMA each with the same
// V operand: a single bf16 rounding of p moves a row's output by up to
// 2^-9 |V|, which for rows that cancel is above the accuracy asked of this
// path; hi + lo carries p to about 2^-17.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>

#include <type_traits>

#include "pkv_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;                      // two 16-column MFMA tiles
constexpr int kRowsPerGroup = kWaves * kRowsPerWave;  // 128 (token, head) rows
constexpr int kKeys = 32;                             // keys per K/V tile

// A tile's row maximum must exceed the reference maximum by more than this
// (log2 units) before that row's accumulators are rescaled; weights <= 2^8.
constexpr float kRescaleSlack = 8.0f;
// A weight of at least this shows that its row's maximum may exceed the
// reference by more than kRescaleSlack (2^8 = 256, less a margin for exp2's
// rounding).
constexpr float kGrowWeight = 255.5f;

// D = A B + C on a 16x16x32 bf16 tile.  Lane l supplies row (l % 16) of A and
// column (l % 16) of B, each as 8 consecutive k-slots of group l / 16; it
// receives D[4 (l / 16) + r][l % 16] in element r.
__device__ inline f32x4_t mfma16x16x32(const uint4& a, const uint4& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even
// (one v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Max / sum over the four 16-lane groups of the wave (lanes with equal
// l % 16), with the VALU row-swap instructions.
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

// LDS row pitch of a staged K or V tile, in 16-bit elements: D plus 8 (16 B)
// of padding, so the 16 rows one MFMA operand read touches start in
// different banks.
template <int D>
struct Pitch {
  static constexpr int kElems = D + 8;
  static constexpr int kTile = kKeys * kElems;  // elements per staged matrix
};

// One thread's share of staging a K/V tile: D / 64 (1 or 2) pieces of 16
// bytes of K and the same of V (a tile is 32 rows of D bf16 = 4 D pieces per
// matrix), and whether each piece's row is live.  Plain members, no arrays:
// the compiler keeps them in registers.  Every load is issued unconditionally
// -- a row that is not live (past the context, or whose block id lies outside
// the pool) reads the first piece of the pool instead and is stored as zeros
// -- so the loads stay in flight across the MFMA work instead of being waited
// for at a branch.
template <int D>
struct Stage {
  static constexpr int kPer = D / 64;
  static constexpr int kChunks = D / 8;  // 16-byte pieces per key row
  static constexpr int kLog2D = D == 128 ? 7 : 6;
  uint4 k0, v0, k1, v1;
  bool ok0, ok1;
  int e0, e1;  // table entries of the next tile to load
};

__device__ inline int stage_key(int u, int chunks) { return (threadIdx.x + kThreads * u) / chunks; }

// Table entries of this thread's rows of key tile `t0` (positions clamped to
// the context, so every read is inside the sequence's row of the table).
template <int D>
__device__ inline void stage_entries(Stage<D>& st, const int32_t* __restrict__ table, int t0,
                                     int n, int log2b) {
  st.e0 = table[min(t0 + stage_key(0, Stage<D>::kChunks), n - 1) >> log2b];
  if constexpr (Stage<D>::kPer == 2)
    st.e1 = table[min(t0 + stage_key(1, Stage<D>::kChunks), n - 1) >> log2b];
}

template <int D>
__device__ inline void stage_piece(uint4& k, uint4& v, bool& ok, int e, int u,
                                   const uint16_t* __restrict__ k_cache,
                                   const uint16_t* __restrict__ v_cache, int t0, int n, int log2b,
                                   int g, int num_kv_heads, int num_blocks) {
  const int idx = threadIdx.x + kThreads * u;
  const int key = idx / Stage<D>::kChunks;
  const int c = idx - key * Stage<D>::kChunks;
  const int t = t0 + key;
  ok = (t < n) & (e >= 0) & (e < num_blocks);
  // (block, head) run index fits 32 bits (num_blocks * num_kv_heads < 2^31,
  // checked by the host); one 64-bit shift-add gives the element offset
  const int run = e * num_kv_heads + g;
  const int64_t off = ((int64_t)run << (log2b + Stage<D>::kLog2D)) +
                      (((t & ((1 << log2b) - 1)) * D) + 8 * c);
  const int64_t at = ok ? off : 0;
  k = *reinterpret_cast<const uint4*>(k_cache + at);
  v = *reinterpret_cast<const uint4*>(v_cache + at);
}

template <int D>
__device__ inline void stage_load(Stage<D>& st, const uint16_t* __restrict__ k_cache,
                                  const uint16_t* __restrict__ v_cache, int t0, int n, int log2b,
                                  int g, int num_kv_heads, int num_blocks) {
  stage_piece<D>(st.k0, st.v0, st.ok0, st.e0, 0, k_cache, v_cache, t0, n, log2b, g, num_kv_heads,
                 num_blocks);
  if constexpr (Stage<D>::kPer == 2)
    stage_piece<D>(st.k1, st.v1, st.ok1, st.e1, 1, k_cache, v_cache, t0, n, log2b, g,
                   num_kv_heads, num_blocks);
}

// x if keep, else zeros: a mask on each 32-bit part (a select of whole
// vectors can turn into a select of their addresses, which sends the staging
// registers to scratch memory).  Only V rows need it: a K row that is not
// live only meets logits the causal mask replaces by -inf (such rows lie past
// every row's position), while its V row is multiplied by weight 0, which
// must not meet NaN or Inf.
__device__ inline uint4 keep_or_zero(uint4 x, bool keep) {
  const uint32_t m = keep ? 0xffffffffu : 0u;
  return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
}

template <int D>
__device__ inline void stage_store(const Stage<D>& st, uint16_t* lk, uint16_t* lv) {
  {
    const int idx = threadIdx.x;
    const int key = idx / Stage<D>::kChunks;
    const int c = idx - key * Stage<D>::kChunks;
    *reinterpret_cast<uint4*>(lk + key * Pitch<D>::kElems + 8 * c) = st.k0;
    *reinterpret_cast<uint4*>(lv + key * Pitch<D>::kElems + 8 * c) = keep_or_zero(st.v0, st.ok0);
  }
  if constexpr (Stage<D>::kPer == 2) {
    const int idx = threadIdx.x + kThreads;
    const int key = idx / Stage<D>::kChunks;
    const int c = idx - key * Stage<D>::kChunks;
    *reinterpret_cast<uint4*>(lk + key * Pitch<D>::kElems + 8 * c) = st.k1;
    *reinterpret_cast<uint4*>(lv + key * Pitch<D>::kElems + 8 * c) = keep_or_zero(st.v1, st.ok1);
  }
}

// ------------------------------------------------------- launch order
//
// A workgroup's run time is proportional to its number of key tiles, which
// depends on the sequence's cached prefix, known only on the device.  The
// workgroups are therefore handed their (sequence, q-tile) items longest
// first: workgroup b takes the item of rank b / Hkv in the order of key-tile
// count descending, ties by item index (s tps + qt), items with nothing to
// do last.  Every workgroup computes the rank selection itself from
// context_lens and query_start_loc: a histogram of the counts in LDS, the
// bin of the rank, then the item inside the bin.  Without it the heavy
// q-tiles of long-prefix sequences could start last and run alone at the
// end of the launch.

constexpr int kOrderBins = 4096;     // histogram bins (counts above are coarsened)
constexpr int kOrderMaxItems = 512;  // beyond: plain order (q-tiles heaviest first)

// Exclusive prefix sum over the workgroup's threads (thread order); also
// returns the total.  Uses `tmp` [kWaves] of LDS; ends with a barrier.
__device__ inline int block_exclusive_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = tmp[w];
    before += w < wave ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + x - v;
}

// Key of item i = s tps + qt: key tiles + 1, or 0 when the q-tile holds no
// new token (the same count the kernel's loop runs).
template <int kTokens>
__device__ inline int item_key(int i, int tiles_per_seq, const int32_t* __restrict__ context_lens,
                               const int32_t* __restrict__ query_start_loc, int max_context_len) {
  const int s = i / tiles_per_seq, qt = i - s * tiles_per_seq;
  const int nnew = query_start_loc[s + 1] - query_start_loc[s];
  const int j0 = qt * kTokens;
  if (j0 >= nnew) return 0;
  const int n = min(context_lens[s], max_context_len);
  const int pmax = n - nnew + min(j0 + kTokens, nnew) - 1;
  return (pmax >= 0 ? (pmax + kKeys) / kKeys : 0) + 1;
}

// The item of rank `rank` (see above); `hist` is kOrderBins + kOrderMaxItems
// ints of LDS (the histogram, then each item's key), `tmp` kWaves + 3 ints.
// All threads of the workgroup call it; items <= kOrderMaxItems.  Its cost
// (two item keys per thread, four barriers and two scans) is what limits the
// item count: every workgroup repeats it.
template <int kTokens>
__device__ int item_of_rank(int rank, int items, int tiles_per_seq,
                            const int32_t* __restrict__ context_lens,
                            const int32_t* __restrict__ query_start_loc, int max_context_len,
                            int* hist, int* tmp) {
  int* keys = hist + kOrderBins;
  // keys lie in [0, max_context_len / kKeys + 2]; coarsen them to the bins
  const int max_key = max_context_len / kKeys + 2;
  int shift = 0;
  while ((max_key >> shift) >= kOrderBins) ++shift;
  for (int b = threadIdx.x; b < kOrderBins; b += kThreads) hist[b] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < items; i += kThreads) {
    const int k = item_key<kTokens>(i, tiles_per_seq, context_lens, query_start_loc,
                                    max_context_len) >> shift;
    keys[i] = k;
    atomicAdd(&hist[k], 1);
  }
  __syncthreads();
  // bin of the rank: bins from the highest down, kOrderBins / kThreads per thread
  constexpr int kPer = kOrderBins / kThreads;
  const int top = kOrderBins - 1 - (int)threadIdx.x * kPer;  // this thread's bins top .. top - kPer + 1
  int mine = 0;
  for (int k = 0; k < kPer; ++k) mine += hist[top - k];
  int total;
  int above = block_exclusive_scan(mine, tmp, total);  // items in higher bins
  if (rank >= above && rank < above + mine) {
    for (int k = 0; k < kPer; ++k) {
      const int c = hist[top - k];
      if (rank < above + c) {
        tmp[kWaves] = top - k;
        tmp[kWaves + 1] = rank - above;  // position inside the bin
        break;
      }
      above += c;
    }
  }
  __syncthreads();
  const int bin = tmp[kWaves], pos = tmp[kWaves + 1];
  // the pos-th item (index order) of that bin: contiguous item ranges per thread
  const int per = (items + kThreads - 1) / kThreads;
  const int i0 = min(items, (int)threadIdx.x * per), i1 = min(items, i0 + per);
  int cnt = 0;
  for (int i = i0; i < i1; ++i) cnt += keys[i] == bin;
  const int before = block_exclusive_scan(cnt, tmp, total);
  if (pos >= before && pos < before + cnt) {
    int k = before;
    for (int i = i0; i < i1; ++i) {
      if (keys[i] != bin) continue;
      if (k == pos) {
        tmp[kWaves + 2] = i;
        break;
      }
      ++k;
    }
  }
  __syncthreads();
  return tmp[kWaves + 2];
}

template <int D, int G>
__global__ __launch_bounds__(kThreads, 3) void prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, int32_t max_blocks_per_seq,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start_loc,
    int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t num_blocks, int32_t log2b, int32_t max_context_len, int32_t tiles_per_seq,
    float qscale) {
  constexpr int kTokens = kRowsPerGroup / G;  // new tokens per workgroup
  constexpr int KK = D / 32;                  // k-steps of the QK product
  constexpr int DT = D / 16;                  // 16-dim tiles of the output

  __shared__ __align__(16) uint16_t lds[2][2][Pitch<D>::kTile];  // [buffer][K, V]

  // Heaviest tiles (last new tokens, most keys) first; the workgroups of one
  // (sequence, KV head) are num_seqs * num_kv_heads apart in launch order.
  // Workgroup b serves KV head b % Hkv (consecutive workgroups go to
  // different XCDs, so each XCD's L2 keeps the K/V of its heads) and the
  // item of rank b / Hkv, longest first.
  const int bid = blockIdx.x;
  const int g = bid % num_kv_heads;
  const int rest = bid / num_kv_heads;
  const int items = num_seqs * tiles_per_seq;
  int s, qt;
  static_assert(sizeof(lds) >= (kOrderBins + kOrderMaxItems) * sizeof(int), "order scratch");
  if (items <= kOrderMaxItems) {
    __shared__ int sm_tmp[kWaves + 3];
    // the histogram and keys live in the staging buffers, unused until the
    // pipeline starts (4608 ints; the smallest staging area holds 4608)
    const int it = item_of_rank<kTokens>(rest, items, tiles_per_seq, context_lens,
                                         query_start_loc, max_context_len,
                                         reinterpret_cast<int*>(&lds[0][0][0]), sm_tmp);
    s = it / tiles_per_seq;
    qt = it - s * tiles_per_seq;
  } else {
    s = rest % num_seqs;
    qt = tiles_per_seq - 1 - rest / num_seqs;
  }

  const int q0 = query_start_loc[s];
  const int q1 = query_start_loc[s + 1];
  const int nnew = q1 - q0;
  const int j0 = qt * kTokens;
  if (j0 >= nnew) return;
  const int n = min(context_lens[s], max_context_len);
  const int first = n - nnew;  // position of new token 0
  const int jend = min(j0 + kTokens, nnew);
  const int pmax = first + jend - 1;
  const int ntiles = pmax >= 0 ? (pmax + kKeys) / kKeys : 0;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int32_t* table = block_tables + (int64_t)s * max_blocks_per_seq;

  // This lane's two rows (one per column tile): token, query head, position.
  int row_tok[2], row_head[2], pos[2];
  bool row_ok[2];
  uint4 qv[2][KK];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = wave * kRowsPerWave + 16 * c + col;
    const int j = j0 + r / G;
    row_tok[c] = q0 + j;
    row_head[c] = g * G + r % G;
    // query_start_loc entries outside [0, num_tokens] break the contract;
    // such rows are neither read nor written
    row_ok[c] = j < jend && q0 + j >= 0 && q0 + j < num_tokens;
    // rows past the tile's tokens act as its last token (their output is
    // dropped), so no row is masked everywhere
    pos[c] = row_ok[c] ? first + j : pmax;
    const uint16_t* qp = q + ((int64_t)row_tok[c] * num_q_heads + row_head[c]) * D + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qv[c][kk] = row_ok[c] ? *reinterpret_cast<const uint4*>(qp + 32 * kk) : make_uint4(0, 0, 0, 0);
  }

  f32x4_t o[2][DT];
  float m[2], lsum[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    m[c] = -INFINITY;
    lsum[c] = 0.0f;
#pragma unroll
    for (int t = 0; t < DT; ++t) o[c][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // Pipeline: table entries two tiles ahead, K/V one tile ahead (registers),
  // the current tile in LDS.  The loads past the last tile read live memory
  // and land in the unused buffer.
  Stage<D> st;
  if (ntiles > 0) {
    stage_entries<D>(st, table, 0, n, log2b);
    stage_load<D>(st, k_cache, v_cache, 0, n, log2b, g, num_kv_heads, num_blocks);
    stage_entries<D>(st, table, kKeys, n, log2b);
    stage_store<D>(st, lds[0][0], lds[0][1]);
  }
  __syncthreads();

  // One key tile; MASKED tiles reach past the workgroup's first position and
  // apply the causal mask, the others (all but the last one or two) skip it.
  auto tile = [&](const int kt, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    const int buf = kt & 1;
    stage_load<D>(st, k_cache, v_cache, (kt + 1) * kKeys, n, log2b, g, num_kv_heads, num_blocks);
    stage_entries<D>(st, table, (kt + 2) * kKeys, n, log2b);
    const uint16_t* lk = lds[buf][0];
    const uint16_t* lv = lds[buf][1];

    // S^T: keys 16 h + 4 grp + r of the tile, rows col of both column tiles.
    f32x4_t sc[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sc[0][h] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      sc[1][h] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // K fragments in order j = h KK + kk, each read two steps before its
    // two MFMAs so the LDS latency overlaps the products of the previous ones.
    auto kread = [&](int j) {
      const int h = j / KK, kk = j % KK;
      return *reinterpret_cast<const uint4*>(lk + (16 * h + col) * Pitch<D>::kElems + 32 * kk +
                                             8 * grp);
    };
    uint4 kf0 = kread(0), kf1 = kread(1);
#pragma unroll
    for (int j = 0; j < 2 * KK; ++j) {
      const uint4 a = kf0;
      kf0 = kf1;
      if (j + 2 < 2 * KK) kf1 = kread(j + 2);
      const int h = j / KK;
      sc[0][h] = mfma16x16x32(a, qv[0][j % KK], sc[0][h]);
      sc[1][h] = mfma16x16x32(a, qv[1][j % KK], sc[1][h]);
    }

    // Online softmax of each row; P^T operands (hi and lo parts) in the S^T
    // key order.
    uint4 pb[2], pl[2];
    const int tbase = kt * kKeys + 4 * grp;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      // raw logits; qscale > 0, so the scaled maximum is qscale * max
      float x[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = tbase + 16 * h + r;
          x[h][r] = sc[c][h][r];
          if constexpr (kMasked) x[h][r] = t <= pos[c] ? x[h][r] : -INFINITY;
        }
      // Weights against the running reference.  The row maximum only matters
      // when it exceeds the reference by more than the slack, and then some
      // weight is at least 2^slack; below a threshold just under that no row
      // can grow, so the maximum is computed only when a weight reaches it
      // (always on the first tile, whose reference is -inf).  The rescale
      // then follows the same test as always, and the weights are recomputed
      // against the new reference: the result is the same bit for bit.
      float p[2][4];
      float pmax = 0.0f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[h][r] = fast_exp2(fmaf(x[h][r], qscale, -m[c]));
          pmax = fmaxf(pmax, p[h][r]);
        }
      if (__builtin_amdgcn_ballot_w64(!(pmax < kGrowWeight))) {
        float mx = -INFINITY;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, x[h][r]);
        mx = rows_max(mx) * qscale;
        const bool grow = mx > m[c] + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float alpha = grow ? fast_exp2(m[c] - mx) : 1.0f;
          if (grow) m[c] = mx;
          lsum[c] *= alpha;
#pragma unroll
          for (int t = 0; t < DT; ++t) o[c][t] *= alpha;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) p[h][r] = fast_exp2(fmaf(x[h][r], qscale, -m[c]));
        }
      }
      uint32_t ph[4], plo[4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const float p0 = p[h][r];
          const float p1 = p[h][r + 1];
          lsum[c] += p0 + p1;
          const uint32_t hp = pack_bf16(p0, p1);
          ph[2 * h + r / 2] = hp;
          plo[2 * h + r / 2] = pack_bf16(p0 - __uint_as_float(hp << 16),
                                         p1 - __uint_as_float(hp & 0xffff0000u));
        }
      pb[c] = make_uint4(ph[0], ph[1], ph[2], ph[3]);
      pl[c] = make_uint4(plo[0], plo[1], plo[2], plo[3]);
    }

    // O^T += V^T P^T.  Transpose reads: within each 16-lane group, lane
    // 4 k + m names row (key) k at dims d0 + 4 m .. + 3, and lane i receives
    // dim d0 + i of the 4 keys; the two reads give keys 4 grp + k and
    // 16 + 4 grp + k, the order of P^T's k-slots.
    const int key_a = 4 * grp + (col >> 2);
    const int dofs = 4 * (col & 3);
    auto vread = [&](int t) {
      const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(lv + key_a * Pitch<D>::kElems + 16 * t + dofs));
      const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(lv + (key_a + 16) * Pitch<D>::kElems + 16 * t + dofs));
      const uint2 a0 = __builtin_bit_cast(uint2, v0);
      const uint2 a1 = __builtin_bit_cast(uint2, v1);
      return make_uint4(a0.x, a0.y, a1.x, a1.y);
    };
    uint4 an = vread(0);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const uint4 a = an;
      if (t + 1 < DT) an = vread(t + 1);
      o[0][t] = mfma16x16x32(a, pb[0], o[0][t]);
      o[1][t] = mfma16x16x32(a, pb[1], o[1][t]);
      o[0][t] = mfma16x16x32(a, pl[0], o[0][t]);
      o[1][t] = mfma16x16x32(a, pl[1], o[1][t]);
    }

    stage_store<D>(st, lds[buf ^ 1][0], lds[buf ^ 1][1]);
    __syncthreads();
  };
  // tiles whose last key is <= the workgroup's first position need no mask
  const int kt_plain = min(ntiles, max(0, (first + j0 + 1) / kKeys));
  int kt = 0;
  for (; kt < kt_plain; ++kt) tile(kt, std::false_type{});
  for (; kt < ntiles; ++kt) tile(kt, std::true_type{});

  // Normalise and store: lane holds dims 16 t + 4 grp + r of its rows.
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const float l = rows_sum(lsum[c]);
    if (!row_ok[c]) continue;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t* op = out + ((int64_t)row_tok[c] * num_q_heads + row_head[c]) * D + 4 * grp;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      uint2 w;
      w.x = pack_bf16(o[c][t][0] * inv, o[c][t][1] * inv);
      w.y = pack_bf16(o[c][t][2] * inv, o[c][t][3] * inv);
      *reinterpret_cast<uint2*>(op + 16 * t) = w;
    }
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

template <int D>
int launch_d(int G, dim3 grid, hipStream_t st, uint16_t* out, const uint16_t* q,
             const uint16_t* kc, const uint16_t* vc, const int32_t* bt, int32_t M,
             const int32_t* ctx, const int32_t* qsl, int32_t S, int32_t T, int32_t hq,
             int32_t hkv, int32_t nb, int32_t log2b, int32_t maxctx, int32_t tps, float qscale) {
#define PKV_PREFILL_CASE(GG)                                                                  \
  case GG:                                                                                    \
    hipLaunchKernelGGL((prefill_kernel<D, GG>), grid, dim3(kThreads), 0, st, out, q, kc, vc, \
                       bt, M, ctx, qsl, S, T, hq, hkv, nb, log2b, maxctx, tps, qscale);       \
    return PKV_OK;
  switch (G) {
    PKV_PREFILL_CASE(1)
    PKV_PREFILL_CASE(2)
    PKV_PREFILL_CASE(4)
    PKV_PREFILL_CASE(8)
    PKV_PREFILL_CASE(16)
    default:
      return pkv__fail(PKV_EUNSUPPORTED, "query heads per KV head %d not in {1, 2, 4, 8, 16}", G);
  }
#undef PKV_PREFILL_CASE
}

}  // namespace

extern "C" int pkv_paged_attention_prefill(
    void* out, const void* q, const void* k_cache, const void* v_cache, const pkv_cache_desc* c,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
    int32_t max_new_tokens, int32_t max_context_len, float scale, void* stream) {
  pkv__clear_error();
  int rc = pkv__check_desc(c);
  if (rc) return rc;
  if (c->dtype != PKV_BF16)
    return pkv__fail(PKV_EUNSUPPORTED, "prefill attention is built for bf16 caches only");
  if (c->head_dim != 64 && c->head_dim != 128)
    return pkv__fail(PKV_EUNSUPPORTED, "prefill head_dim %d not in {64, 128}", c->head_dim);
  const int B = c->block_size;
  if (B != 8 && B != 16 && B != 32)
    return pkv__fail(PKV_EUNSUPPORTED, "prefill block_size %d not in {8, 16, 32}", B);
  if (num_seqs < 0 || num_tokens < 0 || max_new_tokens < 0 || max_context_len < 0 ||
      max_blocks_per_seq < 0)
    return pkv__fail(PKV_EINVAL, "negative size argument");
  if (num_q_heads <= 0 || num_q_heads % c->num_kv_heads != 0)
    return pkv__fail(PKV_EINVAL, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                     num_q_heads, c->num_kv_heads);
  if (max_new_tokens > num_tokens || max_new_tokens > max_context_len)
    return pkv__fail(PKV_EINVAL, "max_new_tokens %d exceeds num_tokens %d or max_context_len %d",
                     max_new_tokens, num_tokens, max_context_len);
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * B)
    return pkv__fail(PKV_EINVAL, "max_context_len %d exceeds the table width %d x block_size %d",
                     max_context_len, max_blocks_per_seq, B);
  if (!(scale > 0.0f) || scale == INFINITY)
    return pkv__fail(PKV_EINVAL, "prefill scale must be finite and positive");
  if ((int64_t)c->num_blocks * c->num_kv_heads > INT32_MAX)
    return pkv__fail(PKV_EUNSUPPORTED, "num_blocks * num_kv_heads exceeds 2^31 - 1");
  if (num_seqs == 0 || num_tokens == 0 || max_new_tokens == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
    return pkv__fail(PKV_EINVAL, "NULL device pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      ((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u) ||
      ((uintptr_t)query_start_loc & 3u))
    return pkv__fail(PKV_EINVAL, "q, out and the caches must be 16-byte aligned, index arrays 4-byte");
  const int G = num_q_heads / c->num_kv_heads;
  if (G > kRowsPerGroup || kRowsPerGroup % G != 0)
    return pkv__fail(PKV_EUNSUPPORTED, "query heads per KV head %d not in {1, 2, 4, 8, 16}", G);
  const int64_t tokens_per_group = kRowsPerGroup / G;
  const int64_t tps = (max_new_tokens + tokens_per_group - 1) / tokens_per_group;
  const int64_t grid = tps * num_seqs * c->num_kv_heads;
  if (grid > INT32_MAX) return pkv__fail(PKV_EINVAL, "prefill grid too large");
  if (pkv__validate_enabled()) {
    // debug: the contract of tables, lengths and row ranges, checked on the host first
    const size_t nt = (size_t)num_seqs * max_blocks_per_seq;
    int32_t* ht = (int32_t*)malloc((nt ? nt : 1) * sizeof(int32_t));
    int32_t* hc = (int32_t*)malloc((size_t)num_seqs * sizeof(int32_t));
    int32_t* hq = (int32_t*)malloc((size_t)(num_seqs + 1) * sizeof(int32_t));
    rc = (ht && hc && hq) ? PKV_OK : pkv__fail(PKV_EINVAL, "out of host memory");
    if (!rc && nt) rc = pkv__copy_to_host(ht, block_tables, nt * sizeof(int32_t), stream);
    if (!rc) rc = pkv__copy_to_host(hc, context_lens, (size_t)num_seqs * sizeof(int32_t), stream);
    if (!rc)
      rc = pkv__copy_to_host(hq, query_start_loc, (size_t)(num_seqs + 1) * sizeof(int32_t), stream);
    if (!rc)
      rc = pkv_validate_prefill(ht, max_blocks_per_seq, hc, hq, num_seqs, num_tokens,
                                max_new_tokens, max_context_len, c);
    free(ht);
    free(hc);
    free(hq);
    if (rc) return rc;
  }
  const int log2b = B == 8 ? 3 : (B == 16 ? 4 : 5);
  const float qscale = scale * 1.4426950408889634f;  // logits in log2 units
  hipStream_t st = (hipStream_t)stream;
  if (c->head_dim == 128)
    rc = launch_d<128>(G, dim3((uint32_t)grid), st, (uint16_t*)out, (const uint16_t*)q,
                       (const uint16_t*)k_cache, (const uint16_t*)v_cache, block_tables,
                       max_blocks_per_seq, context_lens, query_start_loc, num_seqs, num_tokens,
                       num_q_heads, c->num_kv_heads, c->num_blocks, log2b, max_context_len,
                       (int32_t)tps, qscale);
  else
    rc = launch_d<64>(G, dim3((uint32_t)grid), st, (uint16_t*)out, (const uint16_t*)q,
                      (const uint16_t*)k_cache, (const uint16_t*)v_cache, block_tables,
                      max_blocks_per_seq, context_lens, query_start_loc, num_seqs, num_tokens,
                      num_q_heads, c->num_kv_heads, c->num_blocks, log2b, max_context_len,
                      (int32_t)tps, qscale);
  if (rc) return rc;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv__fail(PKV_EHIP, "prefill launch: %s", hipGetErrorString(e));
  return PKV_OK;
}
