// Drives the page allocator (pool.cpp) from a script on stdin, for a host build with AddressSanitizer
// and UndefinedBehaviorSanitizer.  Every operation prints one line: its status, the free count and, for
// operations on a sequence, that sequence's block-table row.  The test feeds the same script to the
// oracle's allocator and compares the lines.
//
//   create N  p_0 .. p_{N-1}      pool of N pages with that free order
//   alloc  S  TOKENS MAX          grow sequence S (rows are MAX pages wide) to cover TOKENS tokens
//   free   S                      return every page of sequence S, forget it
//   raw    K  id_0 .. id_{K-1}    return these page ids as given (error cases: foreign, twice, already free)
//   end
#include <stdio.h>
#include <string.h>

#include <map>
#include <vector>

#include "host.h"

int main() {
  llmdec_config cfg{};
  cfg.n_layers = 1, cfg.hidden = 256, cfg.n_heads = 4, cfg.n_kv_heads = 4, cfg.head_dim = 64;
  cfg.intermediate = 688, cfg.vocab = 1024, cfg.page_size = 16, cfg.rms_eps = 1e-6f, cfg.rope_theta = 1e4f;
  llmdec_kv_pool *pool = nullptr;
  static char dummy[16];  // any non-null base: the allocator never touches device memory
  std::map<int, std::vector<int32_t>> rows;
  std::map<int, int32_t> n_pages;
  char op[16];
  while (scanf("%15s", op) == 1) {
    if (!strcmp(op, "end")) break;
    if (!strcmp(op, "create")) {
      int n;
      if (scanf("%d", &n) != 1) return 2;
      std::vector<int32_t> order(n);
      for (int i = 0; i < n; ++i)
        if (scanf("%d", &order[i]) != 1) return 2;
      const llmdec_status st = llmdec_kv_pool_create(&cfg, dummy, llmdec_kv_pool_bytes(&cfg, n), n, order.data(), &pool);
      printf("create %d free %d\n", (int)st, llmdec_kv_pool_free_count(pool));
    } else if (!strcmp(op, "alloc")) {
      int s, tokens, maxp;
      if (scanf("%d %d %d", &s, &tokens, &maxp) != 3) return 2;
      std::vector<int32_t> &row = rows[s];
      if ((int)row.size() != maxp) row.assign(maxp, -1);
      int32_t np = n_pages[s];
      const llmdec_status st = llmdec_kv_pool_alloc(pool, tokens, row.data(), &np, maxp);
      n_pages[s] = np;
      printf("alloc %d free %d row", (int)st, llmdec_kv_pool_free_count(pool));
      for (int32_t p : row) printf(" %d", p);
      printf("\n");
    } else if (!strcmp(op, "free")) {
      int s;
      if (scanf("%d", &s) != 1) return 2;
      const llmdec_status st = llmdec_kv_pool_free(pool, rows[s].data(), n_pages[s]);
      printf("free %d free %d\n", (int)st, llmdec_kv_pool_free_count(pool));
      rows.erase(s);
      n_pages.erase(s);
    } else if (!strcmp(op, "raw")) {
      int k;
      if (scanf("%d", &k) != 1) return 2;
      std::vector<int32_t> ids(k);
      for (int i = 0; i < k; ++i)
        if (scanf("%d", &ids[i]) != 1) return 2;
      const llmdec_status st = llmdec_kv_pool_free(pool, ids.data(), k);
      printf("raw %d free %d\n", (int)st, llmdec_kv_pool_free_count(pool));
    } else {
      return 2;
    }
  }
  llmdec_kv_pool_destroy(pool);
  return 0;
}
