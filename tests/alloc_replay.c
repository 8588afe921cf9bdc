/* Replays an allocator op stream read from stdin and prints every result, so
 * the allocator can run under AddressSanitizer / UBSan in a plain gcc build.
 * Input lines:  N B perm...  then  add s n | fork p c | append s |
 *               step k s1..sk | free s | table s | prefix |
 *               addt s k t1..tk | appt s t | stept k s1..sk t1..tk |
 *               look k t1..tk | hpool n | sout k s1..sk | sin k s1..sk |
 *               saveload (save the state, destroy the handle, go on with
 *               a handle restored from the saved words)
 * Output: one line per op with the return code and results. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pagedkv.h"

int main(void) {
  int n, b;
  if (scanf("%d %d", &n, &b) != 2) return 2;
  int* perm = malloc(sizeof(int) * n);
  for (int i = 0; i < n; ++i)
    if (scanf("%d", &perm[i]) != 1) return 2;
  pkv_alloc* a = pkv_alloc_create(n, b, perm);
  free(perm);
  if (!a) return 3;
  char op[16];
  while (scanf("%15s", op) == 1) {
    if (strcmp(op, "saveload") == 0) {
      size_t nb = pkv_alloc_save_bytes(a), wr = 0;
      void* buf = malloc(nb ? nb : 8);
      int rc = pkv_alloc_save(a, buf, nb, &wr);
      if (rc == 0) {
        pkv_alloc* r = pkv_alloc_restore(buf, wr);
        if (!r) { printf("saveload restore failed: %s\n", pkv_last_error()); return 4; }
        pkv_alloc_destroy(a);
        a = r;
      }
      free(buf);
      printf("saveload %d\n", rc);
    } else if (strcmp(op, "hpool") == 0) {
      int hn;
      if (scanf("%d", &hn) != 1) return 2;
      printf("hpool %d\n", pkv_alloc_set_host_pool(a, hn, NULL));
    } else if (strcmp(op, "sout") == 0 || strcmp(op, "sin") == 0) {
      int k;
      if (scanf("%d", &k) != 1 || k < 0) return 2;
      int64_t* ids = malloc(sizeof(int64_t) * (k > 0 ? k : 1));
      for (int i = 0; i < k; ++i) { long long x; if (scanf("%lld", &x) != 1) return 2; ids[i] = x; }
      int cap = 0;
      for (int i = 0; i < k; ++i) { int32_t len, nb; if (pkv_seq_info(a, ids[i], &len, &nb) == 0) cap += nb; }
      int32_t* pairs = malloc(sizeof(int32_t) * 2 * (cap > 0 ? cap : 1));
      int32_t np = 0;
      int rc = op[1] == 'o' ? pkv_seq_swap_out(a, ids, k, pairs, cap, &np)
                            : pkv_seq_swap_in(a, ids, k, pairs, cap, &np);
      printf("%s %d", op, rc);
      if (rc == 0) for (int i = 0; i < np; ++i) printf(" %d %d", pairs[2 * i], pairs[2 * i + 1]);
      printf("\n");
      free(ids); free(pairs);
    } else if (strcmp(op, "prefix") == 0) {
      printf("prefix %d\n", pkv_prefix_cache_enable(a));
    } else if (strcmp(op, "addt") == 0) {
      long long s; int k;
      if (scanf("%lld %d", &s, &k) != 2 || k < 0) return 2;
      int32_t* t = malloc(sizeof(int32_t) * (k > 0 ? k : 1));
      for (int i = 0; i < k; ++i) if (scanf("%d", &t[i]) != 1) return 2;
      int64_t* slots = malloc(sizeof(int64_t) * (k > 0 ? k : 1));
      int32_t cached = -7;
      int rc = pkv_seq_add_tokens(a, s, t, k, slots, &cached);
      printf("addt %d", rc);
      if (rc == 0) {
        printf(" %d :", cached);
        for (int i = 0; i < k; ++i) printf(" %lld", (long long)slots[i]);
      }
      printf("\n");
      free(t); free(slots);
    } else if (strcmp(op, "appt") == 0) {
      long long s; int tok; int64_t slot; int32_t cow[2];
      if (scanf("%lld %d", &s, &tok) != 2) return 2;
      int rc = pkv_seq_append_token(a, s, tok, &slot, cow);
      if (rc == 0) printf("appt 0 %lld %d %d\n", (long long)slot, cow[0], cow[1]);
      else printf("appt %d\n", rc);
    } else if (strcmp(op, "stept") == 0) {
      int k;
      if (scanf("%d", &k) != 1 || k < 0) return 2;
      int64_t* ids = malloc(sizeof(int64_t) * (k > 0 ? k : 1));
      int32_t* toks = malloc(sizeof(int32_t) * (k > 0 ? k : 1));
      int64_t* slots = malloc(sizeof(int64_t) * (k > 0 ? k : 1));
      int32_t* pairs = malloc(sizeof(int32_t) * 2 * (k > 0 ? k : 1));
      for (int i = 0; i < k; ++i) { long long x; if (scanf("%lld", &x) != 1) return 2; ids[i] = x; }
      for (int i = 0; i < k; ++i) if (scanf("%d", &toks[i]) != 1) return 2;
      int32_t nc = 0;
      int rc = pkv_step_append_tokens(a, ids, toks, k, slots, pairs, &nc);
      printf("stept %d", rc);
      if (rc == 0) {
        for (int i = 0; i < k; ++i) printf(" %lld", (long long)slots[i]);
        printf(" |");
        for (int i = 0; i < nc; ++i) printf(" %d %d", pairs[2 * i], pairs[2 * i + 1]);
      }
      printf("\n");
      free(ids); free(toks); free(slots); free(pairs);
    } else if (strcmp(op, "look") == 0) {
      int k;
      if (scanf("%d", &k) != 1 || k < 0) return 2;
      int32_t* t = malloc(sizeof(int32_t) * (k > 0 ? k : 1));
      for (int i = 0; i < k; ++i) if (scanf("%d", &t[i]) != 1) return 2;
      int32_t* blocks = malloc(sizeof(int32_t) * (k / b > 0 ? k / b : 1));
      int32_t nb = -1;
      int rc = pkv_prefix_cache_lookup(a, t, k, blocks, &nb);
      printf("look %d", rc);
      if (rc == 0) for (int i = 0; i < nb; ++i) printf(" %d", blocks[i]);
      printf("\n");
      free(t); free(blocks);
    } else if (op[0] == 'a' && op[1] == 'd') {
      long long s; int k;
      if (scanf("%lld %d", &s, &k) != 2) return 2;
      int64_t* slots = malloc(sizeof(int64_t) * (k > 0 ? k : 1));
      int rc = pkv_seq_add(a, s, k, slots);
      printf("add %d", rc);
      if (rc == 0) for (int i = 0; i < k; ++i) printf(" %lld", (long long)slots[i]);
      printf("\n");
      free(slots);
    } else if (op[0] == 'f' && op[1] == 'o') {
      long long p, c;
      if (scanf("%lld %lld", &p, &c) != 2) return 2;
      printf("fork %d\n", pkv_seq_fork(a, p, c));
    } else if (op[0] == 'a') {
      long long s; int64_t slot; int32_t cow[2];
      if (scanf("%lld", &s) != 1) return 2;
      int rc = pkv_seq_append(a, s, &slot, cow);
      if (rc == 0) printf("append 0 %lld %d %d\n", (long long)slot, cow[0], cow[1]);
      else printf("append %d\n", rc);
    } else if (op[0] == 's') {
      int k;
      if (scanf("%d", &k) != 1) return 2;
      int64_t* ids = malloc(sizeof(int64_t) * (k > 0 ? k : 1));
      int64_t* slots = malloc(sizeof(int64_t) * (k > 0 ? k : 1));
      int32_t* pairs = malloc(sizeof(int32_t) * 2 * (k > 0 ? k : 1));
      for (int i = 0; i < k; ++i) { long long x; if (scanf("%lld", &x) != 1) return 2; ids[i] = x; }
      int32_t nc = 0;
      int rc = pkv_step_append(a, ids, k, slots, pairs, &nc);
      printf("step %d", rc);
      if (rc == 0) {
        for (int i = 0; i < k; ++i) printf(" %lld", (long long)slots[i]);
        printf(" |");
        for (int i = 0; i < nc; ++i) printf(" %d %d", pairs[2 * i], pairs[2 * i + 1]);
      }
      printf("\n");
      free(ids); free(slots); free(pairs);
    } else if (op[0] == 'f') {
      long long s;
      if (scanf("%lld", &s) != 1) return 2;
      printf("free %d\n", pkv_seq_free(a, s));
    } else if (op[0] == 't') {
      long long s; int32_t len, nb;
      if (scanf("%lld", &s) != 1) return 2;
      int rc = pkv_seq_info(a, s, &len, &nb);
      int32_t sw = 0;
      if (rc == 0) pkv_seq_swapped(a, s, &sw);
      printf("table %d", rc);
      if (rc == 0 && sw) {
        printf(" %d : swapped", len);
      } else if (rc == 0) {
        int32_t* row = malloc(sizeof(int32_t) * (nb > 0 ? nb : 1));
        int64_t id = s; int32_t l2;
        pkv_build_tables(a, &id, 1, row, nb, &l2);
        printf(" %d :", len);
        for (int i = 0; i < nb; ++i) printf(" %d", row[i]);
        free(row);
      }
      printf("\n");
    } else {
      return 2;
    }
  }
  int32_t* fifo = malloc(sizeof(int32_t) * n);
  int32_t* ref = malloc(sizeof(int32_t) * n);
  int32_t nf;
  pkv_alloc_export(a, fifo, &nf, ref);
  printf("final free");
  for (int i = 0; i < nf; ++i) printf(" %d", fifo[i]);
  printf(" | ref");
  for (int i = 0; i < n; ++i) printf(" %d", ref[i]);
  printf("\n");
  pkv_stats st;
  pkv_alloc_stats(a, &st);
  int32_t* hf = malloc(sizeof(int32_t) * 4096);
  int32_t* hr = malloc(sizeof(int32_t) * 4096);
  int32_t hnf = 0;
  if (pkv_host_pool_export(a, hf, &hnf, NULL) == 0 && hnf > 0) {
    printf("host free");
    for (int i = 0; i < hnf; ++i) printf(" %d", hf[i]);
    printf("\n");
  }
  free(hf); free(hr);
  pkv_prefix_stats ps;
  pkv_prefix_cache_stats(a, &ps);
  if (ps.enabled)
    printf("cache %lld %lld %d %lld\n", (long long)ps.hits, (long long)ps.queries, ps.cached_blocks,
           (long long)ps.evictions);
  free(fifo); free(ref);
  pkv_alloc_destroy(a);
  return 0;
}
