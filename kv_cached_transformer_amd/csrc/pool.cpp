// Host-side paged KV pool: a free-page stack over a caller-owned device buffer.
//
// [E] §3.4 ("为什么要自己动手写一个LLM推理引擎"): the cache is cut into
// fixed-size pages taken from a list of free pages when a request needs them
// and returned when it ends.  The free list here is a stack whose initial
// order is the caller's free_order (first entry handed out first); freed pages
// are pushed in the order given.  Growth is all-or-nothing.
#include <stdlib.h>
#include <string.h>

#include "host.h"

using namespace llmdec;

extern "C" size_t llmdec_kv_pool_bytes(const llmdec_config *cfg, int32_t num_pages) {
  if (!cfg || num_pages < 0) return 0;
  return (size_t)cfg->n_layers * 2 * (size_t)num_pages * cfg->n_kv_heads * kPage * cfg->head_dim * 2;
}

extern "C" llmdec_status llmdec_kv_pool_create(const llmdec_config *cfg, void *dev_base, size_t bytes,
                                               int32_t num_pages, const int32_t *free_order, llmdec_kv_pool **out) {
  if (!out) return set_error(LLMDEC_E_INVALID, "kv_pool_create: out is NULL");
  *out = nullptr;
  llmdec_status st = check_config(cfg, "kv_pool_create");
  if (st != LLMDEC_OK) return st;
  if (!dev_base) return set_error(LLMDEC_E_INVALID, "kv_pool_create: dev_base is NULL");
  if (num_pages <= 0) return set_error(LLMDEC_E_INVALID, "kv_pool_create: num_pages must be > 0, got %d", num_pages);
  size_t need = llmdec_kv_pool_bytes(cfg, num_pages);
  if (bytes < need)
    return set_error(LLMDEC_E_INVALID, "kv_pool_create: buffer holds %zu bytes, %d pages need %zu", bytes,
                     num_pages, need);
  llmdec_kv_pool *p = (llmdec_kv_pool *)calloc(1, sizeof(llmdec_kv_pool));
  int32_t *stack = (int32_t *)malloc(sizeof(int32_t) * (size_t)num_pages);
  uint8_t *is_free = (uint8_t *)calloc((size_t)num_pages, 1);
  if (!p || !stack || !is_free) {
    free(p);
    free(stack);
    free(is_free);
    return set_error(LLMDEC_E_INVALID, "kv_pool_create: host allocation failed for %d pages", num_pages);
  }
  for (int32_t i = 0; i < num_pages; ++i) {
    int32_t pg = free_order ? free_order[i] : i;
    if (pg < 0 || pg >= num_pages || is_free[pg]) {
      free(p);
      free(stack);
      free(is_free);
      return set_error(LLMDEC_E_INVALID, "kv_pool_create: free_order is not a permutation (entry %d = %d)", i, pg);
    }
    is_free[pg] = 1;
    stack[num_pages - 1 - i] = pg;  // first entry of free_order on top
  }
  p->cfg = *cfg;
  p->base = dev_base;
  p->bytes = bytes;
  p->num_pages = num_pages;
  p->stack = stack;
  p->top = num_pages;
  p->is_free = is_free;
  *out = p;
  return clear_error();
}

extern "C" llmdec_status llmdec_kv_pool_alloc(llmdec_kv_pool *pool, int32_t tokens_needed, int32_t *row,
                                              int32_t *n_pages_inout, int32_t max_pages) {
  if (!pool || !row || !n_pages_inout) return set_error(LLMDEC_E_INVALID, "kv_pool_alloc: NULL argument");
  int32_t have = *n_pages_inout;
  if (tokens_needed < 0 || max_pages <= 0 || have < 0 || have > max_pages)
    return set_error(LLMDEC_E_INVALID, "kv_pool_alloc: tokens_needed=%d n_pages=%d max_pages=%d out of range",
                     tokens_needed, have, max_pages);
  int32_t need = (int32_t)(((int64_t)tokens_needed + kPage - 1) / kPage);
  if (need > max_pages)
    return set_error(LLMDEC_E_INVALID, "kv_pool_alloc: %d tokens need %d pages but the row holds %d", tokens_needed,
                     need, max_pages);
  int32_t extra = need - have;
  if (extra <= 0) return clear_error();
  if (extra > pool->top)
    return set_error(LLMDEC_E_NO_PAGES, "kv_pool_alloc: need %d more pages, %d free", extra, pool->top);
  for (int32_t i = 0; i < extra; ++i) {
    int32_t pg = pool->stack[--pool->top];
    pool->is_free[pg] = 0;
    row[have + i] = pg;
  }
  *n_pages_inout = need;
  return clear_error();
}

extern "C" llmdec_status llmdec_kv_pool_free(llmdec_kv_pool *pool, const int32_t *pages, int32_t n) {
  if (!pool || (n > 0 && !pages)) return set_error(LLMDEC_E_INVALID, "kv_pool_free: NULL argument");
  if (n < 0) return set_error(LLMDEC_E_INVALID, "kv_pool_free: n = %d", n);
  // validate everything first so a rejected call changes nothing; pages seen in
  // this call are marked 2 while checking and the marks are undone on exit
  llmdec_status st = LLMDEC_OK;
  int32_t i = 0;
  for (; i < n; ++i) {
    int32_t pg = pages[i];
    if (pg < 0 || pg >= pool->num_pages) {
      st = set_error(LLMDEC_E_INVALID, "kv_pool_free: page %d out of range [0,%d)", pg, pool->num_pages);
      break;
    }
    if (pool->is_free[pg]) {
      st = set_error(LLMDEC_E_INVALID, pool->is_free[pg] == 2 ? "kv_pool_free: page %d listed twice"
                                                             : "kv_pool_free: page %d is already free", pg);
      break;
    }
    pool->is_free[pg] = 2;
  }
  for (int32_t j = 0; j < i; ++j) pool->is_free[pages[j]] = 0;
  if (st != LLMDEC_OK) return st;
  for (int32_t i = 0; i < n; ++i) {
    pool->is_free[pages[i]] = 1;
    pool->stack[pool->top++] = pages[i];
  }
  return clear_error();
}

extern "C" int32_t llmdec_kv_pool_free_count(const llmdec_kv_pool *pool) { return pool ? pool->top : -1; }

extern "C" void *llmdec_kv_pool_device_base(const llmdec_kv_pool *pool) { return pool ? pool->base : nullptr; }

extern "C" void llmdec_kv_pool_destroy(llmdec_kv_pool *pool) {
  if (!pool) return;
  free(pool->stack);
  free(pool->is_free);
  free(pool);
}
