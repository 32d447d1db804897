// Host-only check of the prefix cache over a page pool, built with g++ and
// address/undefined-behaviour sanitizers: random requests that share
// prefixes are matched, grown, inserted, released and evicted; after every
// step the free count plus the references held must account for every page.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "kvp.h"

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                                     \
    }                                                                   \
  } while (0)

int main() {
  std::mt19937 rng(465);
  const int P = 16, NP = 512;
  kvp_pool_desc d{NP, P, 1, 64, KVP_BF16};
  kvp_pool* pool = nullptr;
  CHECK(kvp_pool_create(&d, &pool) == KVP_OK);
  kvp_prefix_cache* cache = nullptr;
  CHECK(kvp_prefix_cache_create(pool, &cache) == KVP_OK);
  std::vector<std::vector<int32_t>> prompts;
  std::vector<std::vector<int32_t>> live;  // block tables of live requests
  for (int step = 0; step < 3000; ++step) {
    std::vector<int32_t> toks;
    if (!prompts.empty() && rng() % 4) {
      const auto& src = prompts[rng() % prompts.size()];
      const int cut = int(rng() % (src.size() + 1));
      toks.assign(src.begin(), src.begin() + cut);
    }
    const int extra = 1 + int(rng() % (3 * P));
    for (int i = 0; i < extra; ++i) toks.push_back(int32_t(rng() % 3));
    const int nb = (int(toks.size()) + P - 1) / P;
    std::vector<int32_t> row(nb, -1);
    int32_t matched = 0;
    CHECK(kvp_prefix_match(cache, toks.data(), int32_t(toks.size()), row.data(), nb, &matched) ==
          KVP_OK);
    kvp_status s = kvp_seq_grow(pool, row.data(), nb, matched * P, int32_t(toks.size()));
    if (s == KVP_E_NOPAGES) {
      int32_t freed = 0;
      CHECK(kvp_prefix_evict(cache, nb, &freed) == KVP_OK);
      s = kvp_seq_grow(pool, row.data(), nb, matched * P, int32_t(toks.size()));
    }
    if (s != KVP_OK) {
      CHECK(s == KVP_E_NOPAGES);
      CHECK(kvp_pages_free(pool, matched, row.data()) == KVP_OK);
    } else {
      CHECK(kvp_prefix_insert(cache, toks.data(), int32_t(toks.size()), row.data()) == KVP_OK);
      live.push_back(row);
      prompts.push_back(toks);
      if (prompts.size() > 64) prompts.erase(prompts.begin());
    }
    if (!live.empty() && (rng() % 3 == 0 || live.size() > 12)) {
      const size_t k = rng() % live.size();
      CHECK(kvp_seq_release(pool, live[k].data(), int32_t(live[k].size())) == KVP_OK);
      live.erase(live.begin() + k);
    }
    // accounting: free pages + pages with a reference = all pages
    int used = 0;
    for (int p = 0; p < NP; ++p) used += kvp_pool_refcount(pool, p) > 0;
    CHECK(kvp_pool_free_count(pool) + used == NP);
    CHECK(kvp_prefix_cache_pages(cache) <= used);
  }
  for (auto& row : live) CHECK(kvp_seq_release(pool, row.data(), int32_t(row.size())) == KVP_OK);
  kvp_prefix_cache_destroy(cache);
  CHECK(kvp_pool_free_count(pool) == NP);
  kvp_pool_destroy(pool);
  std::printf("ok\n");
  return 0;
}
