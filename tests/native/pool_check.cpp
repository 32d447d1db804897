// Host-only check of the page pool (free-list, reference counts, row helpers,
// split planner), built with g++ and address/undefined-behaviour sanitizers.
// Random operation sequences are checked against a shadow model after every
// step; the program prints "ok" and exits 0 when every check holds.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "kvp.h"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                                \
    }                                                              \
  } while (0)

int main() {
  std::mt19937 rng(465);
  kvp_pool_desc d{64, 16, 2, 128, KVP_BF16};
  kvp_pool* p = nullptr;
  CHECK(kvp_pool_create(&d, &p) == KVP_OK);
  std::vector<int> ref(64, 0);
  std::vector<int32_t> held;  // one entry per reference we hold
  for (int step = 0; step < 20000; ++step) {
    const int op = rng() % 3;
    if (op == 0) {
      const int n = rng() % 9;
      std::vector<int32_t> ids(n + 1, -7);
      int free_before = kvp_pool_free_count(p);
      kvp_status s = kvp_pages_alloc(p, n, ids.data());
      if (n > free_before) {
        CHECK(s == KVP_E_NOPAGES);
        CHECK(kvp_pool_free_count(p) == free_before);
      } else {
        CHECK(s == KVP_OK);
        for (int i = 0; i < n; ++i) {
          CHECK(ids[i] >= 0 && ids[i] < 64 && ref[ids[i]] == 0);
          ref[ids[i]] = 1;
          held.push_back(ids[i]);
        }
        CHECK(ids[n] == -7);
      }
    } else if (op == 1 && !held.empty()) {
      const int32_t id = held[rng() % held.size()];
      CHECK(kvp_pages_ref(p, 1, &id) == KVP_OK);
      ++ref[id];
      held.push_back(id);
    } else if (op == 2 && !held.empty()) {
      const size_t k = rng() % held.size();
      const int32_t id = held[k];
      held[k] = held.back();
      held.pop_back();
      CHECK(kvp_pages_free(p, 1, &id) == KVP_OK);
      --ref[id];
    }
    int in_use = 0;
    for (int i = 0; i < 64; ++i) {
      CHECK(kvp_pool_refcount(p, i) == ref[i]);
      in_use += ref[i] > 0;
    }
    CHECK(kvp_pool_free_count(p) == 64 - in_use);
  }
  // over-free in one call is refused and changes nothing
  int32_t fresh;
  while (!held.empty()) {
    int32_t id = held.back();
    held.pop_back();
    CHECK(kvp_pages_free(p, 1, &id) == KVP_OK);
  }
  CHECK(kvp_pool_free_count(p) == 64);
  CHECK(kvp_pages_alloc(p, 1, &fresh) == KVP_OK);
  int32_t twice[2] = {fresh, fresh};
  CHECK(kvp_pages_free(p, 2, twice) == KVP_E_INVAL);
  CHECK(kvp_pool_refcount(p, fresh) == 1);
  int32_t bad = 64;
  CHECK(kvp_pages_free(p, 1, &bad) == KVP_E_INVAL);
  CHECK(kvp_pages_ref(p, 1, &bad) == KVP_E_INVAL);
  CHECK(kvp_pages_free(p, 1, &fresh) == KVP_OK);
  CHECK(kvp_pages_ref(p, 1, &fresh) == KVP_E_INVAL);  // free page cannot be shared

  // row helpers: grow, share a prefix, release
  std::vector<int32_t> a(8, -1), b(8, -1);
  CHECK(kvp_seq_grow(p, a.data(), 8, 0, 33) == KVP_OK);  // 3 pages
  CHECK(a[0] >= 0 && a[1] >= 0 && a[2] >= 0 && a[3] == -1);
  CHECK(kvp_seq_grow(p, a.data(), 8, 33, 48) == KVP_OK);  // still 3 pages
  CHECK(a[3] == -1);
  CHECK(kvp_seq_grow(p, a.data(), 8, 48, 49) == KVP_OK);  // 4th page
  CHECK(a[3] >= 0);
  CHECK(kvp_seq_grow(p, a.data(), 8, 49, 8 * 16 + 1) == KVP_E_INVAL);
  CHECK(kvp_seq_share(p, a.data(), b.data(), 2) == KVP_OK);
  CHECK(b[0] == a[0] && b[1] == a[1] && kvp_pool_refcount(p, a[0]) == 2);
  CHECK(kvp_seq_grow(p, b.data(), 8, 32, 40) == KVP_OK);
  CHECK(b[2] >= 0 && b[2] != a[2]);
  CHECK(kvp_seq_release(p, a.data(), 4) == KVP_OK);
  CHECK(a[0] == -1 && kvp_pool_refcount(p, b[0]) == 1);
  CHECK(kvp_seq_release(p, b.data(), 3) == KVP_OK);
  CHECK(kvp_pool_free_count(p) == 64);

  // planner
  kvp_decode_plan_t plan;
  kvp_pool_desc d3{16384, 16, 8, 128, KVP_BF16};
  CHECK(kvp_decode_plan(&d3, 32, 64, 8192, 0, 256, &plan) == KVP_OK);
  CHECK(plan.num_splits >= 1 && plan.use_mfma == 1);
  CHECK(int64_t(plan.num_splits) * plan.pages_per_split >= 512);
  CHECK(int64_t(plan.num_splits - 1) * plan.pages_per_split < 512);
  CHECK(kvp_decode_plan(&d3, 32, 63, 8192, 0, 256, &plan) == KVP_E_INVAL);
  CHECK(kvp_decode_plan(&d3, 32, 8, 8192, 0, 256, &plan) == KVP_OK && plan.use_mfma == 0);
  kvp_pool_desc bad_desc{16, 24, 1, 128, KVP_BF16};
  CHECK(kvp_pool_create(&bad_desc, &p) == KVP_E_INVAL);
  kvp_pool_destroy(p);
  kvp_pool_destroy(nullptr);
  std::printf("ok\n");
  return 0;
}
