// Host side of the paged KV cache: the pool object, its page free-list and
// reference counts, block-table row helpers, and the decode split planner.
//
// "KV-Cache Optimization Techniques", section "PagedAttention": memory is
// divided into pages of P tokens, each request has a page table, and pages are
// allocated only when needed and freed when the request completes; section
// "Prefix Caching": requests with a common prefix share its pages.  Pages are
// handed out last-freed-first (a stack), so recently used memory is reused.
//
// Plain C++17 with no HIP dependency: it is also built on its own with g++
// and sanitizers for host-only tests.
#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <new>
#include <unordered_map>
#include <vector>

#include "kvp.h"

struct kvp_pool {
  kvp_pool_desc desc;
  std::vector<int32_t> free_stack;  // top = back()
  std::vector<int32_t> refcount;    // per page, 0 = free
};

namespace {

bool desc_valid(const kvp_pool_desc* d) {
  if (!d) return false;
  if (d->num_pages <= 0 || d->num_kv_heads <= 0) return false;
  if (d->page_size != 16 && d->page_size != 32) return false;
  if (d->head_dim != 64 && d->head_dim != 128) return false;
  if (d->dtype != KVP_BF16 && d->dtype != KVP_INT8 && d->dtype != KVP_INT4 &&
      d->dtype != KVP_FP8)
    return false;
  // element offsets must fit in 64 bits comfortably; page offsets in 63 bits
  const double elems = double(d->num_pages) * d->num_kv_heads * d->page_size * d->head_dim;
  return elems < 9.0e18;
}

int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" {

const char* kvp_status_string(kvp_status s) {
  switch (s) {
    case KVP_OK: return "ok";
    case KVP_E_INVAL: return "invalid argument";
    case KVP_E_NOPAGES: return "not enough free pages";
    case KVP_E_UNSUPPORTED: return "unsupported shape or dtype";
    case KVP_E_HIP: return "HIP runtime error";
    case KVP_E_SCRATCH: return "the call needs more device scratch than the library's fixed buffer";
  }
  return "unknown status";
}

kvp_status kvp_pool_bytes(const kvp_pool_desc* desc, size_t* kv_bytes, size_t* meta_bytes) {
  if (!desc_valid(desc)) return KVP_E_INVAL;
  const size_t rows = size_t(desc->num_pages) * desc->num_kv_heads * desc->page_size;
  const size_t bits = desc->dtype == KVP_BF16 ? 16 : (desc->dtype == KVP_INT4 ? 4 : 8);
  if (kv_bytes) *kv_bytes = rows * desc->head_dim * bits / 8;
  if (meta_bytes) *meta_bytes = desc->dtype != KVP_BF16 ? rows * 2 * sizeof(uint16_t) : 0;
  return KVP_OK;
}

kvp_status kvp_pool_create(const kvp_pool_desc* desc, kvp_pool** out) {
  if (!out || !desc_valid(desc)) return KVP_E_INVAL;
  kvp_pool* p = new (std::nothrow) kvp_pool;
  if (!p) return KVP_E_INVAL;
  try {
    p->desc = *desc;
    p->free_stack.resize(desc->num_pages);
    // top of the stack is page 0, so a fresh pool hands out 0, 1, 2, ...
    for (int32_t i = 0; i < desc->num_pages; ++i) p->free_stack[i] = desc->num_pages - 1 - i;
    p->refcount.assign(desc->num_pages, 0);
  } catch (...) {
    delete p;
    return KVP_E_INVAL;
  }
  *out = p;
  return KVP_OK;
}

void kvp_pool_destroy(kvp_pool* pool) { delete pool; }

kvp_status kvp_pool_get_desc(const kvp_pool* pool, kvp_pool_desc* out) {
  if (!pool || !out) return KVP_E_INVAL;
  *out = pool->desc;
  return KVP_OK;
}

int32_t kvp_pool_free_count(const kvp_pool* pool) {
  return pool ? int32_t(pool->free_stack.size()) : -1;
}

int32_t kvp_pool_refcount(const kvp_pool* pool, int32_t page) {
  if (!pool || page < 0 || page >= pool->desc.num_pages) return -1;
  return pool->refcount[page];
}

kvp_status kvp_pages_alloc(kvp_pool* pool, int32_t n, int32_t* out_ids) {
  if (!pool || n < 0 || (n > 0 && !out_ids)) return KVP_E_INVAL;
  if (size_t(n) > pool->free_stack.size()) return KVP_E_NOPAGES;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = pool->free_stack.back();
    pool->free_stack.pop_back();
    pool->refcount[id] = 1;
    out_ids[i] = id;
  }
  return KVP_OK;
}

kvp_status kvp_pages_ref(kvp_pool* pool, int32_t n, const int32_t* ids) {
  if (!pool || n < 0 || (n > 0 && !ids)) return KVP_E_INVAL;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= pool->desc.num_pages || pool->refcount[id] <= 0) return KVP_E_INVAL;
    if (pool->refcount[id] > INT32_MAX - n) return KVP_E_INVAL;
  }
  for (int32_t i = 0; i < n; ++i) ++pool->refcount[ids[i]];
  return KVP_OK;
}

kvp_status kvp_pages_free(kvp_pool* pool, int32_t n, const int32_t* ids) {
  if (!pool || n < 0 || (n > 0 && !ids)) return KVP_E_INVAL;
  // validate everything first: a page listed k times needs k references
  std::unordered_map<int32_t, int32_t> times;
  times.reserve(size_t(n) * 2);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= pool->desc.num_pages) return KVP_E_INVAL;
    if (++times[id] > pool->refcount[id]) return KVP_E_INVAL;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (--pool->refcount[id] == 0) pool->free_stack.push_back(id);
  }
  return KVP_OK;
}

kvp_status kvp_seq_grow(kvp_pool* pool, int32_t* row, int32_t max_blocks, int32_t cur_len,
                        int32_t new_len) {
  if (!pool || !row || max_blocks <= 0 || cur_len < 0 || new_len < cur_len) return KVP_E_INVAL;
  const int32_t P = pool->desc.page_size;
  const int32_t have = ceil_div(cur_len, P);
  const int32_t need = ceil_div(new_len, P);
  if (need > max_blocks) return KVP_E_INVAL;
  if (need == have) return KVP_OK;
  return kvp_pages_alloc(pool, need - have, row + have);
}

kvp_status kvp_seq_share(kvp_pool* pool, const int32_t* src_row, int32_t* dst_row,
                         int32_t n_blocks) {
  if (!pool || !src_row || !dst_row || n_blocks < 0) return KVP_E_INVAL;
  kvp_status s = kvp_pages_ref(pool, n_blocks, src_row);
  if (s != KVP_OK) return s;
  std::copy(src_row, src_row + n_blocks, dst_row);
  return KVP_OK;
}

kvp_status kvp_seq_release(kvp_pool* pool, int32_t* row, int32_t n_blocks) {
  if (!pool || !row || n_blocks < 0) return KVP_E_INVAL;
  kvp_status s = kvp_pages_free(pool, n_blocks, row);
  if (s != KVP_OK) return s;
  std::fill(row, row + n_blocks, -1);
  return KVP_OK;
}

// Pages of a sequence that hold only tokens a sink + window decode drops:
// blocks ceil(sink/P) .. floor((n - window)/P) - 1 ("KV-Cache Optimization
// Techniques", section "Token Eviction Strategies", eq. 5; section "Sliding
// Window Cache", eq. 6: memory stays bounded by the window).  Their references
// are dropped and the entries set to -1; entries already -1 are skipped.
kvp_status kvp_seq_evict_window(kvp_pool* pool, int32_t* row, int32_t max_blocks, int32_t ctx_len,
                                int32_t sink_tokens, int32_t window_tokens) {
  if (!pool || !row || max_blocks <= 0 || ctx_len < 0 || sink_tokens < 0 || window_tokens <= 0)
    return KVP_E_INVAL;
  const int32_t P = pool->desc.page_size;
  if (ceil_div(ctx_len, P) > max_blocks) return KVP_E_INVAL;
  if (int64_t(sink_tokens) + window_tokens >= ctx_len) return KVP_OK;
  const int32_t first = ceil_div(sink_tokens, P);
  const int32_t last = (ctx_len - window_tokens) / P;  // exclusive
  std::vector<int32_t> ids;
  for (int32_t i = first; i < last; ++i)
    if (row[i] >= 0) ids.push_back(row[i]);
  const kvp_status s = kvp_pages_free(pool, int32_t(ids.size()), ids.data());
  if (s != KVP_OK) return s;
  for (int32_t i = first; i < last; ++i) row[i] = -1;
  return KVP_OK;
}

// Split planner.  A workgroup covers one (sequence, KV head) pair and one range
// of logical blocks; its wavefronts share the range page by page.  Measured on
// MI355X, page streaming peaks with about one wavefront per SIMD (four per
// compute unit) and loses bandwidth with every extra split (more partial
// traffic, a merge, shorter streams), so workgroups have four wavefronts and
// the split count is the smallest that gives the chip that many wavefronts:
// S = round(4 * CUs / (pairs * waves)), at least 1, never so large that a
// wavefront streams fewer than four pages.  Splits are single-GPU analogues of
// spreading one sequence's cache over several devices and gathering partial
// results ("KV Cache Optimization" glossary, multi-GPU KV splitting).
kvp_status kvp_decode_plan(const kvp_pool_desc* desc, int32_t num_seqs, int32_t num_q_heads,
                           int32_t max_context_len, int32_t num_splits_req, int32_t num_cus,
                           kvp_decode_plan_t* out) {
  if (!desc_valid(desc) || !out || num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0)
    return KVP_E_INVAL;
  if (num_q_heads % desc->num_kv_heads) return KVP_E_INVAL;
  const int32_t g = num_q_heads / desc->num_kv_heads;
  if (g > 64) return KVP_E_UNSUPPORTED;
  const int32_t P = desc->page_size, D = desc->head_dim;
  const int use_mfma = g >= 4;
  // LDS per wave for the in-workgroup merge: g*D partial outputs plus (m, l)
  // per padded head, plus the vector path's probability broadcast; <= 64 KiB.
  // (The part holds 160 KiB per workgroup, but for g = 32 four waves with
  // fewer splits streamed slower than two waves with more: the 64 KiB cap
  // keeps the occupancy that measured best.)
  const int32_t heads_pad = use_mfma ? ((g + 15) / 16) * 16 : g;
  const int64_t lds_per_wave = (int64_t(g) * D + 2 * heads_pad + (use_mfma ? 0 : g * P)) * 4;
  int32_t waves = 4;
  while (waves > 1 && waves * lds_per_wave > 65536) waves /= 2;
  const int32_t nblk = ceil_div(std::max(max_context_len, 1), P);
  const int64_t items = int64_t(num_seqs) * desc->num_kv_heads;
  int32_t S;
  if (num_splits_req > 0) {
    S = num_splits_req;
  } else {
    const int64_t target_waves = 4 * int64_t(std::max(num_cus, 1));
    const int64_t per_split = std::max<int64_t>(items * waves, 1);
    S = int32_t(std::min<int64_t>((target_waves + per_split / 2) / per_split, 1 << 20));
    const int32_t max_by_work = std::max(1, nblk / (waves * 4));
    S = std::max(1, std::min(S, max_by_work));
  }
  S = std::max(1, std::min(S, nblk));
  const int32_t pps = ceil_div(nblk, S);
  S = ceil_div(nblk, pps);  // drop splits that would cover nothing
  out->num_splits = S;
  out->pages_per_split = pps;
  out->waves_per_group = waves;
  out->use_mfma = use_mfma;
  if (S > 1) {
    const size_t parts = size_t(num_seqs) * num_q_heads * S;
    size_t o_bytes = parts * D * sizeof(float);
    o_bytes = (o_bytes + 255) & ~size_t(255);
    out->workspace_bytes = o_bytes + parts * 2 * sizeof(float);
  } else {
    out->workspace_bytes = 0;
  }
  return KVP_OK;
}

}  // extern "C"
