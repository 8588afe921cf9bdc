/*
 * Host block allocator, error state and host-side contract checks.
 *
 * Plain C11, no HIP: it builds into the shared library with the kernels and,
 * on its own, with gcc for CPU tests and sanitizer runs.
 *
 * The pool follows the pages' description of PagedAttention's memory manager:
 *   - fixed-size physical blocks and a per-sequence block table mapping
 *     logical to physical blocks, with a filled count per block (PagedAttention
 *     blog, 0539edu.com, section 3(3), step 1) Prefill);
 *   - a free list and a reference count per block (weishuz.com Month 2,
 *     section 03 reading (2), section 04);
 *   - lazy allocation: a block is taken when a token crosses into a block not
 *     mapped yet (weishuz.com Month 2, section 02, row "page fault");
 *   - sharing by fork and copy-on-write of a shared, partially filled block
 *     on a divergent write (blog section 4, steps (1) and (2)).
 * Where the pages are silent: the free list is a FIFO (take at the head,
 * return at the tail), a finished sequence releases its blocks last-to-first,
 * a batch step appends in array order and is all-or-nothing.
 *
 * Optional prefix caching (weishuz.com Month 2, section 04, and section 03
 * reading (2): a map from block hash to block, reference counts, LRU
 * eviction, a prefix-aware hash chain):
 *   - the key of a full block is a 64-bit chain hash h_i = H(h_{i-1}, its B
 *     token ids), so equal keys mean equal prefixes up to a collision; a hit
 *     also compares the block's own ids and its parent hash, so a false hit
 *     needs a 64-bit collision of two different prefixes' chain hashes;
 *   - a full block is entered when the tokens that fill it get their slots
 *     (prompt blocks at admission, later blocks by appends that carry ids);
 *     the first block entered under a key keeps it;
 *   - a block whose count drops to 0 keeps its entry and waits in the free
 *     list, which is doubly linked so a hit can take it back out; the free
 *     list hands out its head, evicting the entry of a cached block, so the
 *     least recently released block is evicted first and a referenced one
 *     never is;
 *   - a prompt's lookup walks its full blocks from the first and stops at the
 *     first miss; the prompt takes back its hits, then takes fresh blocks,
 *     then enters its missed full blocks.
 */
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pkv_internal.h"

/* ------------------------------------------------------------------ errors */

static _Thread_local char g_err[512];

int pkv__fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

void pkv__clear_error(void) { g_err[0] = '\0'; }

const char* pkv_last_error(void) { return g_err; }

int pkv__validate_enabled(void) {
  const char* v = getenv("PKV_VALIDATE");
  return v && v[0] && strcmp(v, "0") != 0;
}

int pkv__check_desc(const pkv_cache_desc* c) {
  if (!c) return pkv__fail(PKV_EINVAL, "cache descriptor is NULL");
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->block_size <= 0 || c->head_dim <= 0)
    return pkv__fail(PKV_EINVAL, "cache descriptor has a non-positive size "
                     "(num_blocks=%d num_kv_heads=%d block_size=%d head_dim=%d)",
                     c->num_blocks, c->num_kv_heads, c->block_size, c->head_dim);
  if (c->dtype != PKV_F32 && c->dtype != PKV_BF16)
    return pkv__fail(PKV_EINVAL, "unknown dtype %d", c->dtype);
  return PKV_OK;
}

/* --------------------------------------------------------------- the pool */

typedef struct {
  int64_t id;
  int32_t len;       /* tokens held                                       */
  int32_t nblk;      /* blocks mapped = ceil(len / block_size)             */
  int32_t cap;
  int32_t* blocks;   /* block table, logical -> physical                   */
  uint32_t stamp;    /* last batch step that named this sequence           */
  uint8_t state;     /* 0 empty, 1 live, 2 deleted                         */
  uint8_t tracked;   /* token ids known for every position (prefix cache)  */
  uint8_t swapped;   /* table holds host-pool block ids                     */
  uint64_t chain;    /* chain hash through the last full block             */
  int32_t* toks;     /* ids of the partial last block's tokens, [B]        */
} seq_entry;

struct pkv_alloc {
  int32_t num_blocks;
  int32_t block_size;
  /* free list, doubly linked in release order (-1 ends it) */
  int32_t* nxt;
  int32_t* prv;
  int32_t fhead;
  int32_t ftail;
  int32_t nfree;
  int32_t* ref;
  int32_t* touched;  /* scratch for a step's dry run, capacity num_blocks  */
  seq_entry* tab;    /* open-addressing map seq id -> entry                */
  size_t tcap;       /* power of two                                       */
  size_t nlive;
  size_t nused;      /* live + deleted                                     */
  uint32_t step_no;
  /* prefix cache (all NULL / 0 while disabled) */
  int prefix;
  uint64_t* bkey;    /* chain hash of each cached block                    */
  uint64_t* bpar;    /* chain hash of the prefix before it                 */
  int32_t* btok;     /* [num_blocks][B] ids of each cached block            */
  uint8_t* bcached;
  int32_t* map;      /* linear-probing table of block ids, -1 empty        */
  size_t mcap;       /* power of two >= 2 * num_blocks                     */
  int32_t ncached;
  int64_t hits;
  int64_t queries;
  int64_t evictions;
  /* host pool for swapped-out sequences (0 blocks until set) */
  int32_t hnum;
  int32_t* hfifo;    /* ring buffer of free host ids                        */
  int32_t hhead;
  int32_t hnfree;
  int32_t* href;
  int32_t* dmark;    /* per-block scratch of a swap, all zero between calls */
  int32_t* hmark;
};

static uint64_t mix64(uint64_t x) {
  x ^= x >> 33;
  x *= 0xff51afd7ed558ccdULL;
  x ^= x >> 33;
  x *= 0xc4ceb9fe1a85ec53ULL;
  x ^= x >> 33;
  return x;
}

static seq_entry* find(const pkv_alloc* a, int64_t id) {
  size_t mask = a->tcap - 1;
  for (size_t i = (size_t)mix64((uint64_t)id) & mask;; i = (i + 1) & mask) {
    seq_entry* e = &a->tab[i];
    if (e->state == 0) return NULL;
    if (e->state == 1 && e->id == id) return e;
  }
}

static int rehash(pkv_alloc* a, size_t new_cap) {
  seq_entry* t = (seq_entry*)calloc(new_cap, sizeof(seq_entry));
  if (!t) return pkv__fail(PKV_EINVAL, "out of host memory");
  size_t mask = new_cap - 1;
  for (size_t i = 0; i < a->tcap; ++i) {
    seq_entry* e = &a->tab[i];
    if (e->state != 1) continue;
    size_t j = (size_t)mix64((uint64_t)e->id) & mask;
    while (t[j].state != 0) j = (j + 1) & mask;
    t[j] = *e;
  }
  free(a->tab);
  a->tab = t;
  a->tcap = new_cap;
  a->nused = a->nlive;
  return PKV_OK;
}

/* Insert a fresh entry for `id` (must be absent). */
static seq_entry* insert(pkv_alloc* a, int64_t id) {
  if ((a->nused + 1) * 2 > a->tcap) {
    size_t cap = a->tcap;
    while ((a->nlive + 1) * 4 > cap) cap *= 2;
    if (rehash(a, cap) != PKV_OK) return NULL;
  }
  size_t mask = a->tcap - 1;
  size_t i = (size_t)mix64((uint64_t)id) & mask;
  while (a->tab[i].state == 1) i = (i + 1) & mask;
  seq_entry* e = &a->tab[i];
  if (e->state == 0) a->nused++;
  memset(e, 0, sizeof *e);
  e->id = id;
  e->state = 1;
  a->nlive++;
  return e;
}

static void erase(pkv_alloc* a, seq_entry* e) {
  free(e->blocks);
  e->blocks = NULL;
  free(e->toks);
  e->toks = NULL;
  e->state = 2;
  a->nlive--;
}

static int reserve_blocks(seq_entry* e, int32_t n) {
  if (n <= e->cap) return PKV_OK;
  int32_t cap = e->cap ? e->cap : 4;
  while (cap < n) cap *= 2;
  int32_t* b = (int32_t*)realloc(e->blocks, (size_t)cap * sizeof(int32_t));
  if (!b) return pkv__fail(PKV_EINVAL, "out of host memory");
  e->blocks = b;
  e->cap = cap;
  return PKV_OK;
}

/* ------------------------------------------------------- prefix cache */

static const uint64_t kChainSeed = 0x6a09e667f3bcc908ULL;  /* h_{-1} */
static const uint64_t kGolden = 0x9e3779b97f4a7c15ULL;

/* Chain hash of one full block: parent hash, then the block's ids in order,
 * each folded in through the 64-bit finaliser above. */
static uint64_t chain_hash(uint64_t parent, const int32_t* t, int32_t n) {
  uint64_t h = mix64(parent ^ kGolden);
  for (int32_t i = 0; i < n; ++i) h = mix64(h ^ ((uint64_t)(uint32_t)t[i] + kGolden * (uint64_t)(i + 1)));
  return h;
}

/* Map slot holding the block cached under (key, parent, ids), or the empty
 * slot where the probe ended (*found = 0). */
static size_t map_probe(const pkv_alloc* a, uint64_t key, uint64_t parent, const int32_t* t,
                        int* found) {
  const size_t mask = a->mcap - 1;
  const int32_t B = a->block_size;
  for (size_t i = (size_t)mix64(key) & mask;; i = (i + 1) & mask) {
    int32_t b = a->map[i];
    if (b < 0) {
      *found = 0;
      return i;
    }
    if (a->bkey[b] == key && a->bpar[b] == parent &&
        memcmp(a->btok + (size_t)b * B, t, (size_t)B * sizeof(int32_t)) == 0) {
      *found = 1;
      return i;
    }
  }
}

static int32_t map_find(const pkv_alloc* a, uint64_t key, uint64_t parent, const int32_t* t) {
  int found;
  size_t i = map_probe(a, key, parent, t, &found);
  return found ? a->map[i] : -1;
}

/* Enter block b (full, just filled) under the chain hash of its ids. */
static void cache_enter(pkv_alloc* a, int32_t b, uint64_t key, uint64_t parent, const int32_t* t) {
  int found;
  size_t i = map_probe(a, key, parent, t, &found);
  if (found) return; /* the first block entered under a key keeps it */
  const int32_t B = a->block_size;
  a->map[i] = b;
  a->bkey[b] = key;
  a->bpar[b] = parent;
  memcpy(a->btok + (size_t)b * B, t, (size_t)B * sizeof(int32_t));
  a->bcached[b] = 1;
  a->ncached++;
}

/* Remove block b's entry (linear probing: shift later entries back). */
static void cache_evict(pkv_alloc* a, int32_t b) {
  const size_t mask = a->mcap - 1;
  size_t i = (size_t)mix64(a->bkey[b]) & mask;
  while (a->map[i] != b) i = (i + 1) & mask;
  size_t hole = i;
  for (size_t j = (hole + 1) & mask; a->map[j] >= 0; j = (j + 1) & mask) {
    size_t home = (size_t)mix64(a->bkey[a->map[j]]) & mask;
    /* move map[j] into the hole unless its home lies cyclically in (hole, j] */
    int stays = (hole <= j) ? (home > hole && home <= j) : (home > hole || home <= j);
    if (!stays) {
      a->map[hole] = a->map[j];
      hole = j;
    }
  }
  a->map[hole] = -1;
  a->bcached[b] = 0;
  a->ncached--;
  a->evictions++;
}

/* ----------------------------------------------------------- free list */

static void free_unlink(pkv_alloc* a, int32_t b) {
  int32_t p = a->prv[b], n = a->nxt[b];
  if (p >= 0) a->nxt[p] = n; else a->fhead = n;
  if (n >= 0) a->prv[n] = p; else a->ftail = p;
  a->nxt[b] = a->prv[b] = -1;
  a->nfree--;
}

static void return_block(pkv_alloc* a, int32_t b) {
  a->prv[b] = a->ftail;
  a->nxt[b] = -1;
  if (a->ftail >= 0) a->nxt[a->ftail] = b; else a->fhead = b;
  a->ftail = b;
  a->nfree++;
}

/* Hand out the free-list head; its cached contents, if any, are evicted. */
static int32_t take_block(pkv_alloc* a) {
  int32_t b = a->fhead;
  free_unlink(a, b);
  if (a->prefix && a->bcached[b]) cache_evict(a, b);
  a->ref[b] = 1;
  return b;
}

static int no_blocks(const pkv_alloc* a, int64_t needed) {
  return pkv__fail(PKV_ENOBLOCKS, "failed to allocate %lld blocks: %d free of %d total",
                   (long long)needed, a->nfree, a->num_blocks);
}

pkv_alloc* pkv_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order) {
  pkv__clear_error();
  if (num_blocks <= 0 || block_size <= 0 || block_size > PKV_MAX_BLOCK_SIZE) {
    pkv__fail(PKV_EINVAL, "num_blocks (%d) must be positive and block_size (%d) in 1..%d",
              num_blocks, block_size, PKV_MAX_BLOCK_SIZE);
    return NULL;
  }
  pkv_alloc* a = (pkv_alloc*)calloc(1, sizeof *a);
  if (!a) goto oom;
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->nxt = (int32_t*)malloc((size_t)num_blocks * sizeof(int32_t));
  a->prv = (int32_t*)malloc((size_t)num_blocks * sizeof(int32_t));
  int32_t* order = (int32_t*)malloc((size_t)num_blocks * sizeof(int32_t));
  a->ref = (int32_t*)calloc((size_t)num_blocks, sizeof(int32_t));
  a->touched = (int32_t*)malloc((size_t)num_blocks * sizeof(int32_t));
  a->tcap = 64;
  a->tab = (seq_entry*)calloc(a->tcap, sizeof(seq_entry));
  a->fhead = a->ftail = -1;
  if (!a->nxt || !a->prv || !order || !a->ref || !a->touched || !a->tab) {
    free(order);
    goto oom;
  }
  if (free_order) {
    /* must be a permutation: use ref[] as a seen-mark, then clear it */
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || a->ref[b]) {
        pkv__fail(PKV_EINVAL, "free_order is not a permutation of 0..%d (entry %d = %d)",
                  num_blocks - 1, i, b);
        free(order);
        pkv_alloc_destroy(a);
        return NULL;
      }
      a->ref[b] = 1;
      order[i] = b;
    }
    memset(a->ref, 0, (size_t)num_blocks * sizeof(int32_t));
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) order[i] = i;
  }
  a->nfree = 0;
  for (int32_t i = 0; i < num_blocks; ++i) return_block(a, order[i]);
  free(order);
  return a;
oom:
  pkv__fail(PKV_EINVAL, "out of host memory");
  pkv_alloc_destroy(a);
  return NULL;
}

void pkv_alloc_destroy(pkv_alloc* a) {
  if (!a) return;
  if (a->tab)
    for (size_t i = 0; i < a->tcap; ++i)
      if (a->tab[i].state == 1) {
        free(a->tab[i].blocks);
        free(a->tab[i].toks);
      }
  free(a->tab);
  free(a->nxt);
  free(a->prv);
  free(a->ref);
  free(a->touched);
  free(a->bkey);
  free(a->bpar);
  free(a->btok);
  free(a->bcached);
  free(a->map);
  free(a->hfifo);
  free(a->href);
  free(a->dmark);
  free(a->hmark);
  free(a);
}

int pkv_prefix_cache_enable(pkv_alloc* a) {
  pkv__clear_error();
  if (!a) return pkv__fail(PKV_EINVAL, "allocator handle is NULL");
  if (a->prefix) return PKV_OK;
  if (a->nlive) return pkv__fail(PKV_EINVAL, "prefix caching must be enabled before any sequence is added");
  const size_t n = (size_t)a->num_blocks;
  size_t cap = 16;
  while (cap < 2 * n) cap *= 2;
  a->bkey = (uint64_t*)calloc(n, sizeof(uint64_t));
  a->bpar = (uint64_t*)calloc(n, sizeof(uint64_t));
  a->btok = (int32_t*)calloc(n * (size_t)a->block_size, sizeof(int32_t));
  a->bcached = (uint8_t*)calloc(n, 1);
  a->map = (int32_t*)malloc(cap * sizeof(int32_t));
  if (!a->bkey || !a->bpar || !a->btok || !a->bcached || !a->map) {
    free(a->bkey); free(a->bpar); free(a->btok); free(a->bcached); free(a->map);
    a->bkey = a->bpar = NULL; a->btok = a->map = NULL; a->bcached = NULL;
    return pkv__fail(PKV_EINVAL, "out of host memory");
  }
  for (size_t i = 0; i < cap; ++i) a->map[i] = -1;
  a->mcap = cap;
  a->prefix = 1;
  return PKV_OK;
}

static int64_t slot_of(const pkv_alloc* a, const seq_entry* e, int32_t pos) {
  int32_t B = a->block_size;
  return (int64_t)e->blocks[pos / B] * B + pos % B;
}

int pkv_seq_add(pkv_alloc* a, int64_t seq, int32_t num_tokens, int64_t* slots_out) {
  pkv__clear_error();
  if (!a) return pkv__fail(PKV_EINVAL, "allocator handle is NULL");
  if (num_tokens < 0) return pkv__fail(PKV_EINVAL, "num_tokens %d < 0", num_tokens);
  if (find(a, seq)) return pkv__fail(PKV_EINVAL, "sequence %lld already exists", (long long)seq);
  int32_t B = a->block_size;
  int32_t need = (int32_t)(((int64_t)num_tokens + B - 1) / B);
  if (need > a->nfree) return no_blocks(a, need);
  seq_entry* e = insert(a, seq);
  if (!e) return PKV_EINVAL;
  if (reserve_blocks(e, need) != PKV_OK) {
    erase(a, e);
    return PKV_EINVAL;
  }
  for (int32_t i = 0; i < need; ++i) e->blocks[i] = take_block(a);
  e->nblk = need;
  e->len = num_tokens;
  if (slots_out)
    for (int32_t p = 0; p < num_tokens; ++p) slots_out[p] = slot_of(a, e, p);
  return PKV_OK;
}

/* Walk the prompt's full blocks through the cache: the leading blocks found
 * go to hits[] (at most num_tokens / B), the chain hash through the last
 * full block to *chain_out.  Returns the number of hits. */
static int32_t prefix_walk(const pkv_alloc* a, const int32_t* tokens, int32_t num_tokens,
                           int32_t* hits, uint64_t* chain_out) {
  const int32_t B = a->block_size;
  const int32_t full = num_tokens / B;
  uint64_t h = kChainSeed;
  int32_t nhit = 0;
  int walking = a->prefix;
  for (int32_t i = 0; i < full; ++i) {
    const int32_t* t = tokens + (size_t)i * B;
    uint64_t k = chain_hash(h, t, B);
    if (walking) {
      int32_t b = map_find(a, k, h, t);
      if (b >= 0) hits[nhit++] = b; else walking = 0;
      if (nhit == a->num_blocks) walking = 0; /* hits[] holds num_blocks ids at most */
    }
    h = k;
  }
  *chain_out = h;
  return nhit;
}

int pkv_seq_add_tokens(pkv_alloc* a, int64_t seq, const int32_t* tokens, int32_t num_tokens,
                       int64_t* slots_out, int32_t* num_cached_out) {
  pkv__clear_error();
  if (!a) return pkv__fail(PKV_EINVAL, "allocator handle is NULL");
  if (num_tokens < 0) return pkv__fail(PKV_EINVAL, "num_tokens %d < 0", num_tokens);
  if (num_tokens > 0 && !tokens) return pkv__fail(PKV_EINVAL, "tokens is NULL");
  if (find(a, seq)) return pkv__fail(PKV_EINVAL, "sequence %lld already exists", (long long)seq);
  const int32_t B = a->block_size;
  const int32_t need = (int32_t)(((int64_t)num_tokens + B - 1) / B);
  const int32_t full = num_tokens / B;
  /* hits are staged in the step scratch (capacity num_blocks >= need) */
  int32_t* hits = a->touched;
  uint64_t chain = kChainSeed;
  int32_t nhit = 0;
  if (a->prefix) nhit = prefix_walk(a, tokens, num_tokens, hits, &chain);
  int32_t revived = 0;
  for (int32_t i = 0; i < nhit; ++i) revived += a->ref[hits[i]] == 0;
  const int32_t fresh = need - nhit;
  if ((int64_t)fresh + revived > a->nfree) return no_blocks(a, (int64_t)fresh + revived);
  seq_entry* e = insert(a, seq);
  if (!e) return PKV_EINVAL;
  if (reserve_blocks(e, need) != PKV_OK) {
    erase(a, e);
    return PKV_EINVAL;
  }
  if (a->prefix) {
    e->toks = (int32_t*)malloc((size_t)B * sizeof(int32_t));
    if (!e->toks) {
      erase(a, e);
      return pkv__fail(PKV_EINVAL, "out of host memory");
    }
  }
  /* from here on nothing fails */
  for (int32_t i = 0; i < nhit; ++i) {
    int32_t b = hits[i];
    if (a->ref[b] == 0) free_unlink(a, b);
    a->ref[b]++;
    e->blocks[i] = b;
  }
  for (int32_t i = nhit; i < need; ++i) e->blocks[i] = take_block(a);
  e->nblk = need;
  e->len = num_tokens;
  if (a->prefix) {
    a->queries += full;
    a->hits += nhit;
    uint64_t h = kChainSeed;
    for (int32_t i = 0; i < full; ++i) {
      const int32_t* t = tokens + (size_t)i * B;
      uint64_t k = chain_hash(h, t, B);
      if (i >= nhit) cache_enter(a, e->blocks[i], k, h, t);
      h = k;
    }
    e->tracked = 1;
    e->chain = chain;
    memcpy(e->toks, tokens + (size_t)full * B, (size_t)(num_tokens - full * B) * sizeof(int32_t));
  }
  if (slots_out)
    for (int32_t p = 0; p < num_tokens; ++p) slots_out[p] = slot_of(a, e, p);
  if (num_cached_out) *num_cached_out = nhit * B;
  return PKV_OK;
}

int pkv_prefix_cache_lookup(const pkv_alloc* a, const int32_t* tokens, int32_t num_tokens,
                            int32_t* blocks_out, int32_t* num_blocks_out) {
  pkv__clear_error();
  if (!a) return pkv__fail(PKV_EINVAL, "allocator handle is NULL");
  if (num_tokens < 0 || (num_tokens > 0 && !tokens) || !num_blocks_out)
    return pkv__fail(PKV_EINVAL, "bad lookup arguments");
  if (num_tokens / a->block_size > 0 && !blocks_out)
    return pkv__fail(PKV_EINVAL, "blocks_out is NULL");
  uint64_t chain;
  *num_blocks_out = a->prefix ? prefix_walk(a, tokens, num_tokens, blocks_out, &chain) : 0;
  return PKV_OK;
}

int pkv_prefix_cache_stats(const pkv_alloc* a, pkv_prefix_stats* out) {
  pkv__clear_error();
  if (!a || !out) return pkv__fail(PKV_EINVAL, "NULL argument");
  out->enabled = a->prefix;
  out->cached_blocks = a->ncached;
  out->queries = a->queries;
  out->hits = a->hits;
  out->evictions = a->evictions;
  out->hit_rate = a->queries ? (double)a->hits / (double)a->queries : 0.0;
  return PKV_OK;
}

int pkv_seq_fork(pkv_alloc* a, int64_t parent, int64_t child) {
  pkv__clear_error();
  if (!a) return pkv__fail(PKV_EINVAL, "allocator handle is NULL");
  seq_entry* p = find(a, parent);
  if (!p) return pkv__fail(PKV_EINVAL, "unknown parent sequence %lld", (long long)parent);
  if (p->swapped) return pkv__fail(PKV_EINVAL, "sequence %lld is swapped out", (long long)parent);
  if (find(a, child)) return pkv__fail(PKV_EINVAL, "sequence %lld already exists", (long long)child);
  /* insert may move the table: remember the parent's contents by id */
  seq_entry* c = insert(a, child);
  if (!c) return PKV_EINVAL;
  p = find(a, parent);
  if (reserve_blocks(c, p->nblk) != PKV_OK) {
    erase(a, c);
    return PKV_EINVAL;
  }
  if (p->tracked) {
    c->toks = (int32_t*)malloc((size_t)a->block_size * sizeof(int32_t));
    if (!c->toks) {
      erase(a, c);
      return pkv__fail(PKV_EINVAL, "out of host memory");
    }
    memcpy(c->toks, p->toks, (size_t)a->block_size * sizeof(int32_t));
    c->tracked = 1;
    c->chain = p->chain;
  }
  if (p->nblk) memcpy(c->blocks, p->blocks, (size_t)p->nblk * sizeof(int32_t));
  c->nblk = p->nblk;
  c->len = p->len;
  for (int32_t i = 0; i < p->nblk; ++i) a->ref[p->blocks[i]]++;
  return PKV_OK;
}

/* Blocks one append to `e` takes (0 or 1) given the current counts. */
static int append_needs(const pkv_alloc* a, const seq_entry* e) {
  int32_t pos = e->len, B = a->block_size;
  if (pos % B == 0) return 1;
  return a->ref[e->blocks[pos / B]] > 1;
}

/* Append one token; the caller has checked that a block is available when
 * append_needs() says so.  Writes the slot and the copy pair (or -1, -1).
 * `token` points at the token's id, or is NULL when the id is unknown (the
 * sequence then stops feeding the prefix cache). */
static int append_one(pkv_alloc* a, seq_entry* e, int64_t* slot_out, int32_t* cow,
                      const int32_t* token) {
  int32_t pos = e->len, B = a->block_size;
  cow[0] = -1;
  cow[1] = -1;
  if (pos % B == 0) {
    if (reserve_blocks(e, e->nblk + 1) != PKV_OK) return PKV_EINVAL;
    e->blocks[e->nblk++] = take_block(a);
  } else {
    int32_t last = e->blocks[pos / B];
    if (a->ref[last] > 1) {
      int32_t fresh = take_block(a);
      a->ref[last]--;
      e->blocks[pos / B] = fresh;
      cow[0] = last;
      cow[1] = fresh;
    }
  }
  *slot_out = slot_of(a, e, pos);
  e->len = pos + 1;
  if (!token) {
    e->tracked = 0;
  } else if (e->tracked) {
    e->toks[pos % B] = *token;
    if ((pos + 1) % B == 0) {
      uint64_t k = chain_hash(e->chain, e->toks, B);
      cache_enter(a, e->blocks[pos / B], k, e->chain, e->toks);
      e->chain = k;
    }
  }
  return PKV_OK;
}

static int seq_append(pkv_alloc* a, int64_t seq, int64_t* slot_out, int32_t cow_out[2],
                      const int32_t* token) {
  pkv__clear_error();
  if (!a) return pkv__fail(PKV_EINVAL, "allocator handle is NULL");
  if (!slot_out) return pkv__fail(PKV_EINVAL, "slot_out is NULL");
  seq_entry* e = find(a, seq);
  if (!e) return pkv__fail(PKV_EINVAL, "unknown sequence %lld", (long long)seq);
  if (e->swapped) return pkv__fail(PKV_EINVAL, "sequence %lld is swapped out", (long long)seq);
  if (e->len == INT32_MAX) return pkv__fail(PKV_EINVAL, "sequence %lld is full", (long long)seq);
  if (append_needs(a, e) > a->nfree) return no_blocks(a, 1);
  if (e->len % a->block_size == 0 && reserve_blocks(e, e->nblk + 1) != PKV_OK) return PKV_EINVAL;
  int32_t cow[2];
  int rc = append_one(a, e, slot_out, cow, token);
  if (rc == PKV_OK && cow_out) {
    cow_out[0] = cow[0];
    cow_out[1] = cow[1];
  }
  return rc;
}

int pkv_seq_append(pkv_alloc* a, int64_t seq, int64_t* slot_out, int32_t cow_out[2]) {
  return seq_append(a, seq, slot_out, cow_out, NULL);
}

int pkv_seq_append_token(pkv_alloc* a, int64_t seq, int32_t token, int64_t* slot_out,
                         int32_t cow_out[2]) {
  return seq_append(a, seq, slot_out, cow_out, &token);
}

static int step_append(pkv_alloc* a, const int64_t* seqs, const int32_t* tokens, int32_t n,
                       int64_t* slots_out, int32_t* cow_pairs_out, int32_t* num_cow_out) {
  pkv__clear_error();
  if (!a) return pkv__fail(PKV_EINVAL, "allocator handle is NULL");
  if (n < 0) return pkv__fail(PKV_EINVAL, "n %d < 0", n);
  if (n > 0 && (!seqs || !slots_out || !cow_pairs_out))
    return pkv__fail(PKV_EINVAL, "NULL array argument");
  uint32_t stamp = ++a->step_no;
  if (stamp == 0) { /* wrapped: clear every stamp once */
    for (size_t i = 0; i < a->tcap; ++i) a->tab[i].stamp = 0;
    stamp = a->step_no = 1;
  }
  /* pass 1: ids known and distinct; room in every table */
  for (int32_t i = 0; i < n; ++i) {
    seq_entry* e = find(a, seqs[i]);
    if (!e || e->stamp == stamp || e->swapped)
      return pkv__fail(PKV_EINVAL,
                       "step names an unknown, repeated or swapped-out sequence (%lld at %d)",
                       (long long)seqs[i], i);
    e->stamp = stamp;
    if (e->len == INT32_MAX) return pkv__fail(PKV_EINVAL, "sequence %lld is full", (long long)seqs[i]);
    if (e->len % a->block_size == 0 && reserve_blocks(e, e->nblk + 1) != PKV_OK) return PKV_EINVAL;
  }
  /* pass 2: count blocks, lowering the count of each shared block a copy
   * leaves, then undo those decrements */
  int64_t needed = 0;
  int32_t ntouched = 0;
  for (int32_t i = 0; i < n; ++i) {
    seq_entry* e = find(a, seqs[i]);
    int32_t pos = e->len, B = a->block_size;
    if (pos % B == 0) {
      needed++;
    } else {
      int32_t last = e->blocks[pos / B];
      if (a->ref[last] > 1) {
        needed++;
        a->ref[last]--;
        a->touched[ntouched++] = last;
      }
    }
  }
  for (int32_t i = 0; i < ntouched; ++i) a->ref[a->touched[i]]++;
  if (needed > a->nfree) return no_blocks(a, needed);
  /* pass 3: apply */
  int32_t ncow = 0;
  for (int32_t i = 0; i < n; ++i) {
    seq_entry* e = find(a, seqs[i]);
    int32_t cow[2];
    append_one(a, e, &slots_out[i], cow, tokens ? &tokens[i] : NULL);
    if (cow[0] >= 0) {
      cow_pairs_out[2 * ncow] = cow[0];
      cow_pairs_out[2 * ncow + 1] = cow[1];
      ncow++;
    }
  }
  if (num_cow_out) *num_cow_out = ncow;
  return PKV_OK;
}

int pkv_step_append(pkv_alloc* a, const int64_t* seqs, int32_t n, int64_t* slots_out,
                    int32_t* cow_pairs_out, int32_t* num_cow_out) {
  return step_append(a, seqs, NULL, n, slots_out, cow_pairs_out, num_cow_out);
}

int pkv_step_append_tokens(pkv_alloc* a, const int64_t* seqs, const int32_t* tokens, int32_t n,
                           int64_t* slots_out, int32_t* cow_pairs_out, int32_t* num_cow_out) {
  if (n > 0 && !tokens) {
    pkv__clear_error();
    return pkv__fail(PKV_EINVAL, "tokens is NULL");
  }
  return step_append(a, seqs, tokens, n, slots_out, cow_pairs_out, num_cow_out);
}

/* ------------------------------------------------------------- swapping */

static int32_t host_take(pkv_alloc* a) {
  int32_t h = a->hfifo[a->hhead];
  a->hhead = (a->hhead + 1 == a->hnum) ? 0 : a->hhead + 1;
  a->hnfree--;
  return h;
}

static void host_return(pkv_alloc* a, int32_t h) {
  int64_t tail = (int64_t)a->hhead + a->hnfree;
  if (tail >= a->hnum) tail -= a->hnum;
  a->hfifo[tail] = h;
  a->hnfree++;
}

int pkv_alloc_set_host_pool(pkv_alloc* a, int32_t num_host_blocks, const int32_t* free_order) {
  pkv__clear_error();
  if (!a) return pkv__fail(PKV_EINVAL, "allocator handle is NULL");
  if (a->hnum) return pkv__fail(PKV_EINVAL, "the host pool is already set");
  if (num_host_blocks <= 0) return pkv__fail(PKV_EINVAL, "num_host_blocks %d <= 0", num_host_blocks);
  const size_t n = (size_t)num_host_blocks;
  int32_t* fifo = (int32_t*)malloc(n * sizeof(int32_t));
  int32_t* ref = (int32_t*)calloc(n, sizeof(int32_t));
  int32_t* hmark = (int32_t*)calloc(n, sizeof(int32_t));
  int32_t* dmark = (int32_t*)calloc((size_t)a->num_blocks, sizeof(int32_t));
  if (!fifo || !ref || !hmark || !dmark) {
    free(fifo); free(ref); free(hmark); free(dmark);
    return pkv__fail(PKV_EINVAL, "out of host memory");
  }
  for (int32_t i = 0; i < num_host_blocks; ++i) {
    int32_t h = free_order ? free_order[i] : i;
    if (h < 0 || h >= num_host_blocks || hmark[h]) {
      free(fifo); free(ref); free(hmark); free(dmark);
      return pkv__fail(PKV_EINVAL, "host free_order is not a permutation of 0..%d (entry %d = %d)",
                       num_host_blocks - 1, i, h);
    }
    hmark[h] = 1;
    fifo[i] = h;
  }
  memset(hmark, 0, n * sizeof(int32_t));
  a->hnum = num_host_blocks;
  a->hfifo = fifo;
  a->href = ref;
  a->hmark = hmark;
  a->dmark = dmark;
  a->hhead = 0;
  a->hnfree = num_host_blocks;
  return PKV_OK;
}

/* Move a group of sequences between the pools (out: device -> host).  Each
 * distinct block of the group (first appearance in array, then table order)
 * goes to a block taken from the target pool; pairs_out receives (source,
 * target) ids in that order; the source blocks are released last pair first. */
static int swap_group(pkv_alloc* a, const int64_t* seqs, int32_t n, int32_t* pairs_out,
                      int32_t max_pairs, int32_t* num_pairs_out, int out) {
  pkv__clear_error();
  if (!a) return pkv__fail(PKV_EINVAL, "allocator handle is NULL");
  if (!a->hnum) return pkv__fail(PKV_EINVAL, "no host pool: call pkv_alloc_set_host_pool first");
  if (n < 0 || (n > 0 && (!seqs || !pairs_out)) || !num_pairs_out)
    return pkv__fail(PKV_EINVAL, "bad swap arguments");
  uint32_t stamp = ++a->step_no;
  if (stamp == 0) {
    for (size_t i = 0; i < a->tcap; ++i) a->tab[i].stamp = 0;
    stamp = a->step_no = 1;
  }
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    seq_entry* e = find(a, seqs[i]);
    if (!e || e->stamp == stamp || e->swapped != (out ? 0 : 1))
      return pkv__fail(PKV_EINVAL, "swap names an unknown, repeated or misplaced sequence (%lld at %d)",
                       (long long)seqs[i], i);
    e->stamp = stamp;
    total += e->nblk;
  }
  if (total > max_pairs)
    return pkv__fail(PKV_EINVAL, "pairs_out holds %d pairs, the group maps %lld blocks", max_pairs,
                     (long long)total);
  int32_t* src_ref = out ? a->ref : a->href;
  int32_t* cnt = out ? a->dmark : a->hmark;
  int32_t* order = (int32_t*)malloc((size_t)(total > 0 ? total : 1) * sizeof(int32_t));
  if (!order) return pkv__fail(PKV_EINVAL, "out of host memory");
  int32_t nd = 0;
  for (int32_t i = 0; i < n; ++i) {
    const seq_entry* e = find(a, seqs[i]);
    for (int32_t j = 0; j < e->nblk; ++j) {
      int32_t b = e->blocks[j];
      if (cnt[b]++ == 0) order[nd++] = b;
    }
  }
  int rc = PKV_OK;
  for (int32_t k = 0; k < nd && rc == PKV_OK; ++k)
    if (cnt[order[k]] != src_ref[order[k]])
      rc = pkv__fail(PKV_EINVAL, "block %d is shared with a sequence outside the group", order[k]);
  const int32_t dst_free = out ? a->hnfree : a->nfree;
  if (rc == PKV_OK && nd > dst_free)
    rc = pkv__fail(PKV_ENOBLOCKS, "failed to allocate %d blocks: %d free of %d total", nd, dst_free,
                   out ? a->hnum : a->num_blocks);
  if (rc != PKV_OK) {
    for (int32_t k = 0; k < nd; ++k) cnt[order[k]] = 0;
    free(order);
    return rc;
  }
  /* apply: from here on nothing fails */
  for (int32_t k = 0; k < nd; ++k) {
    const int32_t b = order[k];
    int32_t d;
    if (out) {
      d = host_take(a);
      a->href[d] = a->ref[b];
    } else {
      d = take_block(a);
      a->ref[d] = a->href[b];
    }
    pairs_out[2 * k] = b;
    pairs_out[2 * k + 1] = d;
    cnt[b] = d + 1; /* from now on: where b went */
  }
  for (int32_t k = nd - 1; k >= 0; --k) {
    const int32_t b = order[k];
    if (out) {
      a->ref[b] = 0;
      return_block(a, b);
    } else {
      a->href[b] = 0;
      host_return(a, b);
    }
  }
  for (int32_t i = 0; i < n; ++i) {
    seq_entry* e = find(a, seqs[i]);
    for (int32_t j = 0; j < e->nblk; ++j) e->blocks[j] = cnt[e->blocks[j]] - 1;
    e->swapped = out ? 1 : 0;
  }
  for (int32_t k = 0; k < nd; ++k) cnt[order[k]] = 0;
  free(order);
  *num_pairs_out = nd;
  return PKV_OK;
}

int pkv_seq_swap_out(pkv_alloc* a, const int64_t* seqs, int32_t n, int32_t* pairs_out,
                     int32_t max_pairs, int32_t* num_pairs_out) {
  return swap_group(a, seqs, n, pairs_out, max_pairs, num_pairs_out, 1);
}

int pkv_seq_swap_in(pkv_alloc* a, const int64_t* seqs, int32_t n, int32_t* pairs_out,
                    int32_t max_pairs, int32_t* num_pairs_out) {
  return swap_group(a, seqs, n, pairs_out, max_pairs, num_pairs_out, 0);
}

int pkv_seq_swapped(const pkv_alloc* a, int64_t seq, int32_t* swapped_out) {
  pkv__clear_error();
  if (!a || !swapped_out) return pkv__fail(PKV_EINVAL, "NULL argument");
  const seq_entry* e = find(a, seq);
  if (!e) return pkv__fail(PKV_EINVAL, "unknown sequence %lld", (long long)seq);
  *swapped_out = e->swapped;
  return PKV_OK;
}

int pkv_host_pool_export(const pkv_alloc* a, int32_t* free_fifo_out, int32_t* num_free_out,
                         int32_t* ref_cnt_out) {
  pkv__clear_error();
  if (!a) return pkv__fail(PKV_EINVAL, "allocator handle is NULL");
  if (free_fifo_out)
    for (int32_t i = 0; i < a->hnfree; ++i) {
      int64_t j = (int64_t)a->hhead + i;
      if (j >= a->hnum) j -= a->hnum;
      free_fifo_out[i] = a->hfifo[j];
    }
  if (num_free_out) *num_free_out = a->hnfree;
  if (ref_cnt_out && a->hnum) memcpy(ref_cnt_out, a->href, (size_t)a->hnum * sizeof(int32_t));
  return PKV_OK;
}

int pkv_seq_free(pkv_alloc* a, int64_t seq) {
  pkv__clear_error();
  if (!a) return pkv__fail(PKV_EINVAL, "allocator handle is NULL");
  seq_entry* e = find(a, seq);
  if (!e) return pkv__fail(PKV_EINVAL, "unknown sequence %lld", (long long)seq);
  for (int32_t i = e->nblk - 1; i >= 0; --i) {
    int32_t b = e->blocks[i];
    if (e->swapped) {
      if (--a->href[b] == 0) host_return(a, b);
    } else if (--a->ref[b] == 0) {
      return_block(a, b);
    }
  }
  erase(a, e);
  return PKV_OK;
}

int pkv_seq_info(const pkv_alloc* a, int64_t seq, int32_t* len_out, int32_t* num_blocks_out) {
  pkv__clear_error();
  if (!a) return pkv__fail(PKV_EINVAL, "allocator handle is NULL");
  const seq_entry* e = find(a, seq);
  if (!e) return pkv__fail(PKV_EINVAL, "unknown sequence %lld", (long long)seq);
  if (len_out) *len_out = e->len;
  if (num_blocks_out) *num_blocks_out = e->nblk;
  return PKV_OK;
}

int pkv_build_tables(const pkv_alloc* a, const int64_t* seqs, int32_t n, int32_t* tables_out,
                     int32_t width, int32_t* ctx_lens_out) {
  pkv__clear_error();
  if (!a) return pkv__fail(PKV_EINVAL, "allocator handle is NULL");
  if (n < 0 || width < 0) return pkv__fail(PKV_EINVAL, "negative size (n=%d width=%d)", n, width);
  if (n > 0 && (!seqs || !tables_out || !ctx_lens_out))
    return pkv__fail(PKV_EINVAL, "NULL array argument");
  for (int32_t i = 0; i < n; ++i) {
    const seq_entry* e = find(a, seqs[i]);
    if (!e) return pkv__fail(PKV_EINVAL, "unknown sequence %lld", (long long)seqs[i]);
    if (e->swapped)
      return pkv__fail(PKV_EINVAL, "sequence %lld is swapped out", (long long)seqs[i]);
    if (e->nblk > width)
      return pkv__fail(PKV_EINVAL, "sequence %lld holds %d blocks, more than width %d",
                       (long long)seqs[i], e->nblk, width);
  }
  for (int32_t i = 0; i < n; ++i) {
    const seq_entry* e = find(a, seqs[i]);
    int32_t* row = tables_out + (size_t)i * (size_t)width;
    if (e->nblk) memcpy(row, e->blocks, (size_t)e->nblk * sizeof(int32_t));
    for (int32_t j = e->nblk; j < width; ++j) row[j] = 0;
    ctx_lens_out[i] = e->len;
  }
  return PKV_OK;
}

int pkv_alloc_stats(const pkv_alloc* a, pkv_stats* out) {
  pkv__clear_error();
  if (!a || !out) return pkv__fail(PKV_EINVAL, "NULL argument");
  int32_t B = a->block_size;
  int32_t* fill = (int32_t*)calloc((size_t)a->num_blocks, sizeof(int32_t));
  if (!fill) return pkv__fail(PKV_EINVAL, "out of host memory");
  int64_t logical = 0;
  for (size_t i = 0; i < a->tcap; ++i) {
    const seq_entry* e = &a->tab[i];
    if (e->state != 1 || e->swapped) continue;
    logical += e->len;
    for (int32_t j = 0; j < e->nblk; ++j) {
      int32_t f = e->len - j * B;
      if (f > B) f = B;
      if (f > fill[e->blocks[j]]) fill[e->blocks[j]] = f;
    }
  }
  int64_t filled = 0;
  for (int32_t b = 0; b < a->num_blocks; ++b) filled += fill[b];
  free(fill);
  out->num_blocks = a->num_blocks;
  out->num_free = a->nfree;
  out->block_size = B;
  out->num_seqs = (int32_t)a->nlive;
  out->capacity_tokens = (int64_t)a->num_blocks * B;
  out->allocated_slots = (int64_t)(a->num_blocks - a->nfree) * B;
  out->filled_slots = filled;
  out->logical_tokens = logical;
  out->utilization = out->allocated_slots ? (double)filled / (double)out->allocated_slots : 0.0;
  return PKV_OK;
}

int pkv_alloc_export(const pkv_alloc* a, int32_t* free_fifo_out, int32_t* num_free_out,
                     int32_t* ref_cnt_out) {
  pkv__clear_error();
  if (!a) return pkv__fail(PKV_EINVAL, "allocator handle is NULL");
  if (free_fifo_out) {
    int32_t i = 0;
    for (int32_t b = a->fhead; b >= 0; b = a->nxt[b]) free_fifo_out[i++] = b;
  }
  if (num_free_out) *num_free_out = a->nfree;
  if (ref_cnt_out) memcpy(ref_cnt_out, a->ref, (size_t)a->num_blocks * sizeof(int32_t));
  return PKV_OK;
}

/* ------------------------------------------------------ save / restore */
/*
 * The whole allocator state as a flat array of int64 words (uint64 hashes
 * stored as their bit patterns):
 *   [0] magic  [1] version  [2] num_blocks  [3] block_size  [4] prefix on
 *   [5] host blocks  [6] free blocks  [7] live sequences  [8] cached blocks
 *   [9] hits  [10] queries  [11] evictions  [12] free host blocks
 *   free list, head to tail                         (free blocks words)
 *   reference counts                                (num_blocks words)
 *   per live sequence, ids ascending: id, length, blocks, flags (1 tracked,
 *     2 swapped), chain hash, the block table, then block_size token ids
 *     when tracked (the partial last block's ids first)
 *   per cached block, ids ascending: block, key, parent key, its token ids
 *   free host list, head to tail; host reference counts
 * Scratch (step stamps, marks) is not state: a restored handle behaves as
 * the saved one on every later call.
 */
enum { kSaveHeader = 13 };
static const int64_t kSaveMagic = 0x4554415453564B50LL; /* "PKVSTATE" */
static const int64_t kSaveVersion = 1;

static int cmp_i64(const void* x, const void* y) {
  const int64_t a = *(const int64_t*)x, b = *(const int64_t*)y;
  return (a > b) - (a < b);
}

static size_t save_words(const pkv_alloc* a) {
  size_t w = kSaveHeader + (size_t)a->nfree + (size_t)a->num_blocks;
  for (size_t i = 0; i < a->tcap; ++i) {
    const seq_entry* e = &a->tab[i];
    if (e->state != 1) continue;
    w += 5 + (size_t)e->nblk + (e->tracked ? (size_t)a->block_size : 0);
  }
  if (a->prefix) w += (size_t)a->ncached * (3 + (size_t)a->block_size);
  w += (size_t)a->hnfree + (size_t)a->hnum;
  return w;
}

size_t pkv_alloc_save_bytes(const pkv_alloc* a) {
  pkv__clear_error();
  if (!a) {
    pkv__fail(PKV_EINVAL, "allocator handle is NULL");
    return 0;
  }
  return save_words(a) * sizeof(int64_t);
}

int pkv_alloc_seq_ids(const pkv_alloc* a, int64_t* ids_out, int32_t max_ids, int32_t* num_out) {
  pkv__clear_error();
  if (!a || !num_out || max_ids < 0 || (max_ids > 0 && !ids_out))
    return pkv__fail(PKV_EINVAL, "bad argument");
  if ((size_t)max_ids < a->nlive)
    return pkv__fail(PKV_EINVAL, "%zu live sequences, room for %d", a->nlive, max_ids);
  int32_t k = 0;
  for (size_t i = 0; i < a->tcap; ++i)
    if (a->tab[i].state == 1) ids_out[k++] = a->tab[i].id;
  qsort(ids_out, (size_t)k, sizeof(int64_t), cmp_i64);
  *num_out = k;
  return PKV_OK;
}

int pkv_alloc_save(const pkv_alloc* a, void* buf, size_t bytes, size_t* written) {
  pkv__clear_error();
  if (!a || (!buf && bytes)) return pkv__fail(PKV_EINVAL, "bad argument");
  const size_t need = save_words(a);
  if (bytes < need * sizeof(int64_t))
    return pkv__fail(PKV_EINVAL, "buffer of %zu bytes, the state needs %zu", bytes,
                     need * sizeof(int64_t));
  int64_t* ids = (int64_t*)malloc((a->nlive ? a->nlive : 1) * sizeof(int64_t));
  if (!ids) return pkv__fail(PKV_EINVAL, "out of host memory");
  int32_t nseq = 0;
  pkv_alloc_seq_ids(a, ids, (int32_t)a->nlive, &nseq);
  int64_t* w = (int64_t*)buf;
  const int32_t B = a->block_size;
  size_t k = 0;
  w[k++] = kSaveMagic;
  w[k++] = kSaveVersion;
  w[k++] = a->num_blocks;
  w[k++] = B;
  w[k++] = a->prefix;
  w[k++] = a->hnum;
  w[k++] = a->nfree;
  w[k++] = nseq;
  w[k++] = a->prefix ? a->ncached : 0;
  w[k++] = a->hits;
  w[k++] = a->queries;
  w[k++] = a->evictions;
  w[k++] = a->hnfree;
  for (int32_t b = a->fhead; b >= 0; b = a->nxt[b]) w[k++] = b;
  for (int32_t b = 0; b < a->num_blocks; ++b) w[k++] = a->ref[b];
  for (int32_t i = 0; i < nseq; ++i) {
    const seq_entry* e = find(a, ids[i]);
    w[k++] = e->id;
    w[k++] = e->len;
    w[k++] = e->nblk;
    w[k++] = (e->tracked ? 1 : 0) | (e->swapped ? 2 : 0);
    w[k++] = e->tracked ? (int64_t)e->chain : 0; /* unused once ids are unknown */
    for (int32_t j = 0; j < e->nblk; ++j) w[k++] = e->blocks[j];
    if (e->tracked)
      for (int32_t j = 0; j < B; ++j) w[k++] = e->toks[j];
  }
  free(ids);
  if (a->prefix)
    for (int32_t b = 0; b < a->num_blocks; ++b) {
      if (!a->bcached[b]) continue;
      w[k++] = b;
      w[k++] = (int64_t)a->bkey[b];
      w[k++] = (int64_t)a->bpar[b];
      for (int32_t j = 0; j < B; ++j) w[k++] = a->btok[(size_t)b * B + j];
    }
  for (int32_t i = 0; i < a->hnfree; ++i) {
    int64_t j = (int64_t)a->hhead + i;
    if (j >= a->hnum) j -= a->hnum;
    w[k++] = a->hfifo[j];
  }
  for (int32_t h = 0; h < a->hnum; ++h) w[k++] = a->href[h];
  if (written) *written = k * sizeof(int64_t);
  return PKV_OK;
}

/* restore: reading words with bounds and range checks */
typedef struct {
  const int64_t* w;
  size_t n, k;
  int bad;
} reader;

static int64_t rd(reader* r, int64_t lo, int64_t hi) {
  if (r->bad || r->k >= r->n) {
    r->bad = 1;
    return lo;
  }
  const int64_t x = r->w[r->k++];
  if (x < lo || x > hi) {
    r->bad = 1;
    return lo;
  }
  return x;
}

pkv_alloc* pkv_alloc_restore(const void* buf, size_t bytes) {
  pkv__clear_error();
  if (!buf || bytes % sizeof(int64_t) || bytes < kSaveHeader * sizeof(int64_t)) {
    pkv__fail(PKV_EINVAL, "saved state of %zu bytes is not a whole state", bytes);
    return NULL;
  }
  reader r = {(const int64_t*)buf, bytes / sizeof(int64_t), 0, 0};
  if (rd(&r, kSaveMagic, kSaveMagic) != kSaveMagic || r.bad ||
      rd(&r, kSaveVersion, kSaveVersion) != kSaveVersion || r.bad) {
    pkv__fail(PKV_EINVAL, "not a saved allocator state (magic or version)");
    return NULL;
  }
  const int32_t N = (int32_t)rd(&r, 1, INT32_MAX);
  const int32_t B = (int32_t)rd(&r, 1, INT32_MAX);
  const int prefix = (int)rd(&r, 0, 1);
  const int32_t H = (int32_t)rd(&r, 0, INT32_MAX);
  const int32_t nfree = (int32_t)rd(&r, 0, N);
  const int64_t nseq = rd(&r, 0, INT32_MAX);
  const int32_t ncached = (int32_t)rd(&r, 0, N);
  /* counters below 2^62 leave every later increment room */
  const int64_t kCounterMax = (int64_t)1 << 62;
  const int64_t hits = rd(&r, 0, kCounterMax);
  const int64_t queries = rd(&r, 0, kCounterMax);
  const int64_t evictions = rd(&r, 0, kCounterMax);
  const int32_t hnfree = (int32_t)rd(&r, 0, H);
  /* every device and host block's reference count is one word of the state,
   * so the pools cannot be larger than the words present */
  if (r.bad || (!prefix && ncached) || hits > queries || B > PKV_MAX_BLOCK_SIZE ||
      (int64_t)N + H > (int64_t)r.n) {
    pkv__fail(PKV_EINVAL, "saved state has a bad header");
    return NULL;
  }
  pkv_alloc* a = pkv_alloc_create(N, B, NULL);
  if (!a) return NULL;
  int32_t* count = (int32_t*)calloc((size_t)N, sizeof(int32_t));
  int32_t* hcount = (int32_t*)calloc(H ? (size_t)H : 1, sizeof(int32_t));
  const char* why = NULL;
  if (!count || !hcount) {
    why = "out of host memory";
    goto fail;
  }
  if (prefix && pkv_prefix_cache_enable(a) != PKV_OK) {
    why = "out of host memory";
    goto fail;
  }
  if (H && pkv_alloc_set_host_pool(a, H, NULL) != PKV_OK) {
    why = "out of host memory";
    goto fail;
  }
  /* free list: relink in the saved order */
  a->fhead = a->ftail = -1;
  a->nfree = 0;
  for (int32_t i = 0; i < N; ++i) a->nxt[i] = a->prv[i] = -1;
  for (int32_t i = 0; i < nfree; ++i) {
    const int32_t b = (int32_t)rd(&r, 0, N - 1);
    if (r.bad || count[b]) {
      why = "free list: block out of range or listed twice";
      goto fail;
    }
    count[b] = 1;
    return_block(a, b);
  }
  memset(count, 0, (size_t)N * sizeof(int32_t));
  for (int32_t b = 0; b < N; ++b) a->ref[b] = (int32_t)rd(&r, 0, INT32_MAX);
  if (r.bad) {
    why = "bad reference count";
    goto fail;
  }
  int64_t prev_id = 0;
  for (int64_t i = 0; i < nseq; ++i) {
    const int64_t id = rd(&r, INT64_MIN, INT64_MAX);
    const int32_t len = (int32_t)rd(&r, 0, INT32_MAX);
    const int32_t nblk = (int32_t)rd(&r, 0, INT32_MAX);
    const int flags = (int)rd(&r, 0, 3);
    const uint64_t chain = (uint64_t)rd(&r, INT64_MIN, INT64_MAX);
    if (r.bad || (i > 0 && id <= prev_id) || nblk != (int32_t)(((int64_t)len + B - 1) / B) ||
        ((flags & 1) && !prefix) || ((flags & 2) && !H)) {
      why = "bad sequence record (order, length, block count or flags)";
      goto fail;
    }
    prev_id = id;
    seq_entry* e = insert(a, id);
    if (!e || reserve_blocks(e, nblk) != PKV_OK) {
      why = "out of host memory";
      goto fail;
    }
    e->len = len;
    e->nblk = nblk;
    e->swapped = (flags & 2) ? 1 : 0;
    const int32_t lim = e->swapped ? H : N;
    for (int32_t j = 0; j < nblk; ++j) {
      const int32_t b = (int32_t)rd(&r, 0, lim - 1);
      if (r.bad) {
        why = "block table entry out of range";
        goto fail;
      }
      e->blocks[j] = b;
      if (e->swapped) hcount[b]++; else count[b]++;
    }
    if (flags & 1) {
      e->toks = (int32_t*)malloc((size_t)B * sizeof(int32_t));
      if (!e->toks) {
        why = "out of host memory";
        goto fail;
      }
      for (int32_t j = 0; j < B; ++j) e->toks[j] = (int32_t)rd(&r, INT32_MIN, INT32_MAX);
      e->tracked = 1;
      e->chain = chain;
    }
  }
  for (int32_t b = 0; b < N; ++b)
    if (a->ref[b] != count[b] || (a->ref[b] == 0) != (a->prv[b] >= 0 || a->fhead == b)) {
      why = "reference counts disagree with the block tables or the free list";
      goto fail;
    }
  if (a->nfree != nfree) {
    why = "free list length";
    goto fail;
  }
  for (int32_t i = 0; i < ncached; ++i) {
    const int32_t b = (int32_t)rd(&r, 0, N - 1);
    const uint64_t key = (uint64_t)rd(&r, INT64_MIN, INT64_MAX);
    const uint64_t par = (uint64_t)rd(&r, INT64_MIN, INT64_MAX);
    if (r.bad || a->bcached[b]) {
      why = "cached block out of range or listed twice";
      goto fail;
    }
    for (int32_t j = 0; j < B; ++j)
      a->btok[(size_t)b * B + j] = (int32_t)rd(&r, INT32_MIN, INT32_MAX);
    int found;
    const size_t slot = map_probe(a, key, par, a->btok + (size_t)b * B, &found);
    if (r.bad || found) {
      why = "cached block entry repeated";
      goto fail;
    }
    a->map[slot] = b;
    a->bkey[b] = key;
    a->bpar[b] = par;
    a->bcached[b] = 1;
    a->ncached++;
  }
  a->hits = hits;
  a->queries = queries;
  a->evictions = evictions;
  if (H) {
    memset(a->hmark, 0, (size_t)H * sizeof(int32_t));
    for (int32_t i = 0; i < hnfree; ++i) {
      const int32_t h = (int32_t)rd(&r, 0, H - 1);
      if (r.bad || a->hmark[h]) {
        why = "host free list: block out of range or listed twice";
        goto fail;
      }
      a->hmark[h] = 1;
      a->hfifo[i] = h;
    }
    a->hhead = 0;
    a->hnfree = hnfree;
    for (int32_t h = 0; h < H; ++h) {
      a->href[h] = (int32_t)rd(&r, 0, INT32_MAX);
      if (r.bad || a->href[h] != hcount[h] || (a->href[h] == 0) != (a->hmark[h] == 1)) {
        why = "host reference counts disagree with the tables or the host free list";
        goto fail;
      }
    }
    memset(a->hmark, 0, (size_t)H * sizeof(int32_t));
  }
  if (r.k != r.n) {
    why = "trailing words after the saved state";
    goto fail;
  }
  free(count);
  free(hcount);
  return a;
fail:
  free(count);
  free(hcount);
  pkv_alloc_destroy(a);
  pkv__fail(PKV_EINVAL, "saved allocator state rejected: %s", why ? why : "truncated");
  return NULL;
}

/* ------------------------------------------------------ contract checks */

int pkv_validate_write(const int64_t* slot_mapping, int32_t num_tokens, const pkv_cache_desc* c) {
  pkv__clear_error();
  int rc = pkv__check_desc(c);
  if (rc) return rc;
  if (num_tokens < 0 || (num_tokens > 0 && !slot_mapping))
    return pkv__fail(PKV_EINVAL, "bad slot_mapping argument");
  int64_t nslots = (int64_t)c->num_blocks * c->block_size;
  uint8_t* seen = (uint8_t*)calloc((size_t)nslots, 1);
  if (!seen) return pkv__fail(PKV_EINVAL, "out of host memory");
  for (int32_t t = 0; t < num_tokens; ++t) {
    int64_t s = slot_mapping[t];
    if (s < 0 || s >= nslots) continue;
    if (seen[s]) {
      free(seen);
      return pkv__fail(PKV_ERANGE, "slot %lld of token %d is also named by an earlier token",
                       (long long)s, t);
    }
    seen[s] = 1;
  }
  free(seen);
  return PKV_OK;
}

int pkv_validate_copy(const int32_t* pairs, int32_t num_pairs, const pkv_cache_desc* c) {
  pkv__clear_error();
  int rc = pkv__check_desc(c);
  if (rc) return rc;
  if (num_pairs < 0 || (num_pairs > 0 && !pairs))
    return pkv__fail(PKV_EINVAL, "bad pairs argument");
  uint8_t* role = (uint8_t*)calloc((size_t)c->num_blocks, 1); /* bit0 src, bit1 dst */
  if (!role) return pkv__fail(PKV_EINVAL, "out of host memory");
  for (int32_t i = 0; i < num_pairs; ++i) {
    int32_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s < 0 || s >= c->num_blocks || d < 0 || d >= c->num_blocks) {
      free(role);
      return pkv__fail(PKV_ERANGE, "pair %d (%d, %d) is outside [0, %d)", i, s, d, c->num_blocks);
    }
    role[s] |= 1;
  }
  for (int32_t i = 0; i < num_pairs; ++i) {
    int32_t d = pairs[2 * i + 1];
    if (role[d] & 1) {
      free(role);
      return pkv__fail(PKV_ERANGE, "pair %d: destination %d is also a source", i, d);
    }
    if (role[d] & 2) {
      free(role);
      return pkv__fail(PKV_ERANGE, "pair %d: destination %d repeats", i, d);
    }
    role[d] |= 2;
  }
  free(role);
  return PKV_OK;
}

int pkv_validate_decode(const int32_t* block_tables, int32_t width, const int32_t* context_lens,
                        int32_t num_seqs, int32_t max_context_len, const pkv_cache_desc* c) {
  pkv__clear_error();
  int rc = pkv__check_desc(c);
  if (rc) return rc;
  if (num_seqs < 0 || width < 0 || (num_seqs > 0 && (!block_tables || !context_lens)))
    return pkv__fail(PKV_EINVAL, "bad table arguments");
  int32_t B = c->block_size;
  for (int32_t s = 0; s < num_seqs; ++s) {
    int32_t n = context_lens[s];
    if (n < 0 || n > max_context_len)
      return pkv__fail(PKV_ERANGE, "context_lens[%d] = %d is outside [0, %d]", s, n, max_context_len);
    int32_t nb = (int32_t)(((int64_t)n + B - 1) / B);
    if (nb > width)
      return pkv__fail(PKV_ERANGE, "sequence %d needs %d table entries, width is %d", s, nb, width);
    for (int32_t i = 0; i < nb; ++i) {
      int32_t b = block_tables[(size_t)s * (size_t)width + i];
      if (b < 0 || b >= c->num_blocks)
        return pkv__fail(PKV_ERANGE, "block_tables[%d][%d] = %d is outside [0, %d)", s, i, b,
                         c->num_blocks);
    }
  }
  return PKV_OK;
}

int pkv_validate_prefill(const int32_t* block_tables, int32_t width, const int32_t* context_lens,
                         const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                         int32_t max_new_tokens, int32_t max_context_len, const pkv_cache_desc* c) {
  pkv__clear_error();
  if (num_seqs < 0 || num_tokens < 0 || (num_seqs >= 0 && !query_start_loc))
    return pkv__fail(PKV_EINVAL, "bad query_start_loc arguments");
  if (query_start_loc[0] != 0)
    return pkv__fail(PKV_ERANGE, "query_start_loc[0] = %d, not 0", query_start_loc[0]);
  for (int32_t s = 0; s < num_seqs; ++s) {
    int32_t a = query_start_loc[s], b = query_start_loc[s + 1];
    if (b < a || b > num_tokens)
      return pkv__fail(PKV_ERANGE, "query_start_loc[%d] = %d after %d (num_tokens %d)", s + 1, b,
                       a, num_tokens);
    if (b - a > max_new_tokens)
      return pkv__fail(PKV_ERANGE, "sequence %d has %d new tokens > max_new_tokens %d", s, b - a,
                       max_new_tokens);
    if (context_lens && b - a > context_lens[s])
      return pkv__fail(PKV_ERANGE, "sequence %d has %d new tokens but context %d", s, b - a,
                       context_lens[s]);
  }
  return pkv_validate_decode(block_tables, width, context_lens, num_seqs, max_context_len, c);
}
