/*
 * Fuzz of pkv_alloc_restore, for a sanitizer build (AddressSanitizer and
 * UndefinedBehaviorSanitizer, CPU only).
 *
 * Reads a saved allocator state (the int64 words pkv_alloc_save writes) from
 * a file and hands the library seeded mutations of it: a word set to an
 * extreme or nearby value, a word inserted, dropped or swapped with another,
 * the buffer cut at any byte.  Every result must be either NULL (a state the
 * library refuses) or a handle that behaves as a consistent allocator:
 *   - its own saved state restores again to the same words;
 *   - its counters, free lists and sequence ids can be read;
 *   - every live sequence's table can be built, and one token appended;
 *   - once every sequence is freed, every device and host block is free.
 * A parser that reads past the buffer, trusts a count it has not checked or
 * accepts counts that disagree with its tables ends the run with a sanitizer
 * report or a failed check (exit status 1).
 *
 * Usage: alloc_restore_fuzz <state file> <seed> <iterations>
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pagedkv.h"

static uint64_t rng_state;

static uint64_t next_u64(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545F4914F6CDD1DULL;
}

static int64_t pick_value(int64_t old) {
  switch (next_u64() % 9) {
    case 0: return 0;
    case 1: return -1;
    case 2: return 1;
    case 3: return INT64_MAX;
    case 4: return INT64_MIN;
    case 5: return (int64_t)INT32_MAX + 1;
    case 6: return (int64_t)((uint64_t)old + next_u64() % 5 - 2); /* wraps, no overflow */
    case 7: return (int64_t)(next_u64() % 64);
    default: return (int64_t)next_u64();
  }
}

#define CHECK(cond, what)                                   \
  do {                                                      \
    if (!(cond)) {                                          \
      fprintf(stderr, "iteration %d: %s\n", iter, what);    \
      exit(1);                                              \
    }                                                       \
  } while (0)

/* Drive an accepted handle through the checks above; destroys it. */
static void exercise(pkv_alloc* a, int iter) {
  size_t n = pkv_alloc_save_bytes(a);
  CHECK(n > 0, "save_bytes of an accepted state is 0");
  unsigned char* s1 = (unsigned char*)malloc(n);
  size_t w = 0;
  CHECK(s1 && pkv_alloc_save(a, s1, n, &w) == PKV_OK && w == n && n >= 6 * 8, "save failed");
  int64_t host_blocks;
  memcpy(&host_blocks, s1 + 5 * 8, 8); /* header word 5: host blocks */
  pkv_alloc* b = pkv_alloc_restore(s1, n);
  CHECK(b, "a state the library saved is refused");
  CHECK(pkv_alloc_save_bytes(b) == n, "resaved size differs");
  unsigned char* s2 = (unsigned char*)malloc(n);
  CHECK(s2 && pkv_alloc_save(b, s2, n, &w) == PKV_OK && memcmp(s1, s2, n) == 0,
        "resaved words differ");
  pkv_alloc_destroy(b);
  free(s2);
  free(s1);

  pkv_stats st;
  CHECK(pkv_alloc_stats(a, &st) == PKV_OK, "stats failed");
  int32_t nb = st.num_blocks;
  int32_t* fifo = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nb > 0 ? nb : 1));
  int32_t* ref = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nb > 0 ? nb : 1));
  int32_t nfree = 0;
  CHECK(fifo && ref && pkv_alloc_export(a, fifo, &nfree, ref) == PKV_OK, "export failed");

  int32_t ns = st.num_seqs;
  int64_t* ids = (int64_t*)malloc(sizeof(int64_t) * (size_t)(ns > 0 ? ns : 1));
  int32_t got = -1;
  CHECK(ids && pkv_alloc_seq_ids(a, ids, ns, &got) == PKV_OK && got == ns, "seq_ids failed");
  int32_t* table = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nb > 0 ? nb : 1));
  for (int32_t i = 0; i < ns; ++i) {
    int32_t len = -1, nblk = -1, swapped = 0;
    CHECK(pkv_seq_info(a, ids[i], &len, &nblk) == PKV_OK, "seq_info of a listed id failed");
    CHECK(len >= 0 && nblk >= 0 && nblk <= nb, "seq_info out of range");
    CHECK(pkv_seq_swapped(a, ids[i], &swapped) == PKV_OK, "seq_swapped failed");
    if (swapped) continue;
    int32_t ctx = -1;
    CHECK(pkv_build_tables(a, &ids[i], 1, table, nb > 0 ? nb : 1, &ctx) == PKV_OK && ctx == len,
          "build_tables failed");
    for (int32_t j = 0; j < nblk; ++j) CHECK(table[j] >= 0 && table[j] < nb, "table entry out of range");
    int64_t slot;
    int32_t cow[2];
    const int rc = pkv_seq_append_token(a, ids[i], 1, &slot, cow);
    CHECK(rc == PKV_OK || rc == PKV_ENOBLOCKS || rc == PKV_EINVAL, "append failed oddly");
  }
  for (int32_t i = 0; i < ns; ++i) CHECK(pkv_seq_free(a, ids[i]) == PKV_OK, "free failed");
  CHECK(pkv_alloc_stats(a, &st) == PKV_OK && st.num_seqs == 0, "stats after freeing");
  CHECK(pkv_alloc_export(a, fifo, &nfree, ref) == PKV_OK && nfree == nb, "blocks still held");
  for (int32_t j = 0; j < nb; ++j) CHECK(ref[j] == 0, "reference left after freeing");
  int32_t hn = -1;
  CHECK(pkv_host_pool_export(a, NULL, &hn, NULL) == PKV_OK && hn == host_blocks,
        "host blocks still held");
  free(table);
  free(ids);
  free(ref);
  free(fifo);
  pkv_alloc_destroy(a);
}

int main(int argc, char** argv) {
  if (argc != 4) {
    fprintf(stderr, "usage: %s <state file> <seed> <iterations>\n", argv[0]);
    return 2;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 2;
  fseek(f, 0, SEEK_END);
  const long size = ftell(f);
  fseek(f, 0, SEEK_SET);
  if (size <= 0 || size % 8) return 2;
  const size_t nw = (size_t)size / 8;
  int64_t* orig = (int64_t*)malloc((size_t)size);
  if (!orig || fread(orig, 1, (size_t)size, f) != (size_t)size) return 2;
  fclose(f);
  rng_state = 0x9E3779B97F4A7C15ULL ^ (uint64_t)strtoull(argv[2], NULL, 10);
  const int iters = atoi(argv[3]);
  int accepted = 0;
  for (int iter = 0; iter < iters; ++iter) {
    /* room for the inserted words (at most one per mutation) */
    const size_t cap = (nw + 4) * sizeof(int64_t);
    int64_t* w = (int64_t*)malloc(cap);
    memcpy(w, orig, nw * sizeof(int64_t));
    size_t bytes = nw * sizeof(int64_t);
    const int nmut = 1 + (int)(next_u64() % 3);
    for (int m = 0; m < nmut; ++m) {
      const size_t cur = bytes / 8;
      if (cur == 0) break;
      const size_t k = (size_t)(next_u64() % cur);
      switch (next_u64() % 6) {
        case 0:
        case 1: w[k] = pick_value(w[k]); break;
        case 2: bytes = (size_t)(next_u64() % (bytes + 1)); break;
        case 3:
          if (bytes + 8 <= cap - 8) {
            memmove(w + k + 1, w + k, (cur - k) * sizeof(int64_t));
            w[k] = pick_value(w[k]);
            bytes += 8;
          }
          break;
        case 4:
          memmove(w + k, w + k + 1, (cur - k - 1) * sizeof(int64_t));
          bytes -= 8;
          break;
        default: {
          const size_t k2 = (size_t)(next_u64() % cur);
          const int64_t t = w[k];
          w[k] = w[k2];
          w[k2] = t;
        }
      }
    }
    /* an exact-size copy, so that a read past the end is caught */
    unsigned char* buf = (unsigned char*)malloc(bytes ? bytes : 1);
    memcpy(buf, w, bytes);
    free(w);
    pkv_alloc* a = pkv_alloc_restore(buf, bytes);
    free(buf);
    if (a) {
      ++accepted;
      exercise(a, iter);
    }
  }
  /* the unmutated state must be accepted */
  pkv_alloc* a = pkv_alloc_restore(orig, nw * sizeof(int64_t));
  if (!a) {
    fprintf(stderr, "the original state is refused\n");
    return 1;
  }
  exercise(a, -1);
  free(orig);
  printf("%d of %d mutated states accepted\n", accepted, iters);
  return 0;
}
