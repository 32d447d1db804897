// Host prefix cache over a page pool, and copy-on-write for shared pages.
//
// "KV-Cache Optimization Techniques", section "Prefix Caching": requests that
// share a prefix (system prompt, few-shot examples, documents) reuse its
// KV-cache: the token sequence is hashed, an existing prefix is reused by
// copy-on-write, and cached prefixes are organised in a radix tree for
// longest-prefix matching ("KV Cache" glossary: prefixes keyed at token
// level).  Memory for N requests of T tokens sharing P_shared of them drops
// from N*T*c to P_shared*c + N*(T - P_shared)*c (eq. 2).
//
// The tree's unit is a full page: a node is one block of P token ids, its
// key a 64-bit hash chained over the whole prefix up to and including the
// block, and it holds the physical page with that block's K/V plus one
// reference to it.  Matching walks whole blocks from the root, comparing the
// token ids of every block it accepts (a hash collision can only shorten a
// match, never return wrong pages).  Eviction removes least-recently-used
// leaves whose page no sequence holds any more.
//
// Plain C++17 with no HIP dependency (built with g++ and sanitizers too).
#include <algorithm>
#include <cstdint>
#include <memory>
#include <new>
#include <queue>
#include <unordered_map>
#include <vector>

#include "kvp.h"

namespace {

struct Node {
  uint64_t key = 0;
  std::vector<int32_t> tokens;  // the block's page_size token ids
  int32_t page = -1;
  uint64_t last_use = 0;
  Node* parent = nullptr;
  std::unordered_map<uint64_t, std::unique_ptr<Node>> children;
};

// splitmix64 finalizer: a well-mixed 64-bit function of its input.
uint64_t mix64(uint64_t x) {
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}

// Key of a block given the key of the prefix before it: every token of the
// prefix takes part, so equal keys mean equal prefixes up to collisions.
uint64_t block_key(uint64_t parent_key, const int32_t* tokens, int32_t n) {
  uint64_t h = mix64(parent_key ^ 0x6b76705f70726566ull);
  for (int32_t i = 0; i < n; ++i) h = mix64(h ^ uint64_t(uint32_t(tokens[i])));
  return h;
}

bool same_tokens(const Node& n, const int32_t* tokens, int32_t count) {
  return std::equal(n.tokens.begin(), n.tokens.end(), tokens, tokens + count);
}

}  // namespace

struct kvp_prefix_cache {
  kvp_pool* pool = nullptr;
  int32_t page_size = 0;
  Node root;
  uint64_t tick = 0;
  int32_t pages = 0;
};

namespace {

// Release every page reference below (and including) node; delete children.
void release_subtree(kvp_prefix_cache* c, Node* node) {
  for (auto& kv : node->children) release_subtree(c, kv.second.get());
  node->children.clear();
  if (node->page >= 0) {
    kvp_pages_free(c->pool, 1, &node->page);
    node->page = -1;
    --c->pages;
  }
}

}  // namespace

extern "C" {

kvp_status kvp_prefix_cache_create(kvp_pool* pool, kvp_prefix_cache** out) {
  kvp_pool_desc d;
  if (!out || kvp_pool_get_desc(pool, &d) != KVP_OK) return KVP_E_INVAL;
  kvp_prefix_cache* c = new (std::nothrow) kvp_prefix_cache;
  if (!c) return KVP_E_INVAL;
  c->pool = pool;
  c->page_size = d.page_size;
  *out = c;
  return KVP_OK;
}

void kvp_prefix_cache_destroy(kvp_prefix_cache* cache) {
  if (!cache) return;
  release_subtree(cache, &cache->root);
  delete cache;
}

int32_t kvp_prefix_cache_pages(const kvp_prefix_cache* cache) {
  return cache ? cache->pages : -1;
}

kvp_status kvp_prefix_match(kvp_prefix_cache* cache, const int32_t* tokens, int32_t n_tokens,
                            int32_t* pages_out, int32_t max_pages, int32_t* n_blocks_out) {
  if (!cache || n_tokens < 0 || max_pages < 0 || !n_blocks_out) return KVP_E_INVAL;
  if ((n_tokens > 0 && !tokens) || (max_pages > 0 && !pages_out)) return KVP_E_INVAL;
  const int32_t P = cache->page_size;
  std::vector<Node*> path;
  Node* node = &cache->root;
  for (int32_t blk = 0; (blk + 1) * int64_t(P) <= n_tokens && blk < max_pages; ++blk) {
    const int32_t* t = tokens + int64_t(blk) * P;
    auto it = node->children.find(block_key(node->key, t, P));
    if (it == node->children.end() || !same_tokens(*it->second, t, P)) break;
    node = it->second.get();
    path.push_back(node);
  }
  const int32_t n = int32_t(path.size());
  for (int32_t i = 0; i < n; ++i) pages_out[i] = path[i]->page;
  if (n > 0) {
    const kvp_status s = kvp_pages_ref(cache->pool, n, pages_out);
    if (s != KVP_OK) return s;
  }
  const uint64_t now = ++cache->tick;
  for (Node* p : path) p->last_use = now;
  *n_blocks_out = n;
  return KVP_OK;
}

kvp_status kvp_prefix_insert(kvp_prefix_cache* cache, const int32_t* tokens, int32_t n_tokens,
                             const int32_t* pages) {
  if (!cache || n_tokens < 0 || (n_tokens > 0 && (!tokens || !pages))) return KVP_E_INVAL;
  const int32_t P = cache->page_size;
  const int32_t full = n_tokens / P;
  // Walk the cached part first; the rest are new nodes.  Validate the new
  // nodes' pages before changing anything (all or nothing).
  Node* node = &cache->root;
  int32_t blk = 0;
  for (; blk < full; ++blk) {
    const int32_t* t = tokens + int64_t(blk) * P;
    auto it = node->children.find(block_key(node->key, t, P));
    if (it == node->children.end()) break;
    if (!same_tokens(*it->second, t, P)) return KVP_OK;  // collision: cache nothing more
    node = it->second.get();
  }
  for (int32_t i = blk; i < full; ++i)
    if (kvp_pool_refcount(cache->pool, pages[i]) <= 0) return KVP_E_INVAL;
  for (int32_t i = blk; i < full; ++i)
    for (int32_t j = blk; j < i; ++j)
      if (pages[i] == pages[j]) return KVP_E_INVAL;
  if (full > blk) {
    const kvp_status s = kvp_pages_ref(cache->pool, full - blk, pages + blk);
    if (s != KVP_OK) return s;
  }
  const uint64_t now = ++cache->tick;
  Node* walk = &cache->root;
  for (int32_t i = 0; i < full; ++i) {
    const int32_t* t = tokens + int64_t(i) * P;
    const uint64_t key = block_key(walk->key, t, P);
    auto it = walk->children.find(key);
    if (it == walk->children.end()) {
      auto child = std::make_unique<Node>();
      child->key = key;
      child->tokens.assign(t, t + P);
      child->page = pages[i];
      child->parent = walk;
      it = walk->children.emplace(key, std::move(child)).first;
      ++cache->pages;
    }
    it->second->last_use = now;
    walk = it->second.get();
  }
  return KVP_OK;
}

kvp_status kvp_prefix_evict(kvp_prefix_cache* cache, int32_t n_pages, int32_t* n_freed) {
  if (!cache || n_pages < 0) return KVP_E_INVAL;
  int32_t freed = 0;
  // Leaves whose page only the cache holds, least recently used first; a
  // parent whose last child goes becomes a candidate in turn.
  using Item = std::pair<uint64_t, Node*>;
  std::priority_queue<Item, std::vector<Item>, std::greater<Item>> heap;
  std::vector<Node*> stack{&cache->root};
  while (!stack.empty()) {
    Node* n = stack.back();
    stack.pop_back();
    for (auto& kv : n->children) stack.push_back(kv.second.get());
    if (n != &cache->root && n->children.empty() && kvp_pool_refcount(cache->pool, n->page) == 1)
      heap.emplace(n->last_use, n);
  }
  while (freed < n_pages && !heap.empty()) {
    Node* n = heap.top().second;
    heap.pop();
    Node* parent = n->parent;
    kvp_pages_free(cache->pool, 1, &n->page);
    --cache->pages;
    ++freed;
    parent->children.erase(n->key);  // destroys n
    if (parent != &cache->root && parent->children.empty() &&
        kvp_pool_refcount(cache->pool, parent->page) == 1)
      heap.emplace(parent->last_use, parent);
  }
  if (n_freed) *n_freed = freed;
  return KVP_OK;
}

kvp_status kvp_seq_prepare_append(kvp_pool* pool, int32_t* row, int32_t max_blocks,
                                  int32_t cur_len, int32_t new_len, int32_t* copy_src,
                                  int32_t* copy_dst, int32_t* n_copies) {
  kvp_pool_desc d;
  if (kvp_pool_get_desc(pool, &d) != KVP_OK || !row || max_blocks <= 0 || cur_len < 0 ||
      new_len < cur_len || !n_copies)
    return KVP_E_INVAL;
  const int32_t P = d.page_size;
  const int32_t have = (cur_len + P - 1) / P;
  const int32_t need = (new_len + P - 1) / P;
  if (need > max_blocks) return KVP_E_INVAL;
  for (int32_t i = 0; i < have; ++i)
    if (kvp_pool_refcount(pool, row[i]) <= 0) return KVP_E_INVAL;
  // The only existing block that receives new rows is the partly filled last
  // one; if another sequence (or the prefix cache) also holds it, this
  // sequence gets a private copy first.
  const bool cow = new_len > cur_len && cur_len % P != 0 &&
                   kvp_pool_refcount(pool, row[have - 1]) > 1;
  if (cow && (!copy_src || !copy_dst)) return KVP_E_INVAL;
  const int32_t fresh = need - have;
  if (kvp_pool_free_count(pool) < fresh + (cow ? 1 : 0)) return KVP_E_NOPAGES;
  if (fresh > 0) {
    const kvp_status s = kvp_pages_alloc(pool, fresh, row + have);
    if (s != KVP_OK) return s;
  }
  *n_copies = 0;
  if (cow) {
    int32_t page = -1;
    kvp_status s = kvp_pages_alloc(pool, 1, &page);
    if (s != KVP_OK) return s;  // cannot happen: the free count was checked
    copy_src[0] = row[have - 1];
    copy_dst[0] = page;
    s = kvp_pages_free(pool, 1, &row[have - 1]);
    if (s != KVP_OK) return s;
    row[have - 1] = page;
    *n_copies = 1;
  }
  return KVP_OK;
}

}  // extern "C"
