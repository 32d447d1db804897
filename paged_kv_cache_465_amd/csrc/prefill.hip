// Multi-query paged attention (chunked prefill, verification of drafted
// tokens): host side of the C ABI (argument checks, tiling, launches).  The
// kernel is in prefill_kernels.h; the instances of each KV format are
// compiled in a file of their own, prefill_<format>.hip.
#include <algorithm>
#include <cmath>
#include <vector>

#include "prefill_kernels.h"

namespace kvp {
#define KVP_PREFILL_FMT_EXTERN(F)                                                         \
  extern template hipError_t launch_prefill_fmt<F>(const PrefillArgs&, int, int, int, bool, \
                                                   dim3, hipStream_t);
KVP_PREFILL_FMT_EXTERN(kBF16)
KVP_PREFILL_FMT_EXTERN(kI8)
KVP_PREFILL_FMT_EXTERN(kI4)
KVP_PREFILL_FMT_EXTERN(kFP8)
#undef KVP_PREFILL_FMT_EXTERN
}  // namespace kvp

namespace {

// Tiling of a multi-query call (the natural grid): shape checks shared by the
// launch and the schedule builder.
struct Geometry {
  int g = 0, nt = 0;
  bool quant = false, split = false;
  int64_t rows_wg = 0, tiles = 0, items = 0, wgs = 0;
};

kvp_status prefill_geometry(const kvp_pool_desc& d, int32_t num_seqs, int32_t num_q_heads,
                            int32_t max_blocks, int32_t max_q_len, int32_t max_context_len,
                            Geometry* o) {
  using namespace kvp;
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks <= 0 || max_q_len < 0) return KVP_E_INVAL;
  if (num_q_heads % d.num_kv_heads) return KVP_E_INVAL;
  if (int64_t(max_blocks) * d.page_size > 0x7fffffff) return KVP_E_INVAL;
  if (max_context_len < 0 || int64_t(max_context_len) > int64_t(max_blocks) * d.page_size)
    return KVP_E_INVAL;
  o->g = num_q_heads / d.num_kv_heads;
  if (o->g > 64) return KVP_E_UNSUPPORTED;
  o->quant = d.dtype != KVP_BF16;
  // rows per wavefront: 32 when the longest chunk has at least that many rows;
  // chunks whose rows fit one wavefront split the pages across the four
  const int64_t max_rows = int64_t(max_q_len) * o->g;
  o->split = max_rows <= 32;
  // row-tiled mode: 128 rows per workgroup (bfloat16: the LDS-staged kernel;
  // quantized pools: 32 rows per wavefront when the longest chunk has at least
  // 128 rows, else 16)
  o->nt = o->split ? (max_rows > 16 ? 2 : 1) : (max_rows >= 32 * 4 || !o->quant ? 2 : 1);
  o->rows_wg = o->split ? 16 * o->nt : (o->quant ? 4 * 16 * o->nt : 32 * kFaWaves * kFaRowTiles);
  o->tiles = (max_rows + o->rows_wg - 1) / o->rows_wg;
  o->items = int64_t(num_seqs) * d.num_kv_heads;
  o->wgs = (o->items + 7) / 8 * 8 * o->tiles;
  if (o->tiles > 0x7fffffff || o->wgs > 0x7fffffff) return KVP_E_UNSUPPORTED;
  return KVP_OK;
}

kvp_status prefill_run(const kvp_pool* pool, const void* q, const int32_t* q_start,
                       const void* k_pool, const void* v_pool, const void* k_meta,
                       const void* v_meta, const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                       int32_t max_q_len, int32_t max_context_len, float scale,
                       const int32_t* order, int64_t order_len, void* out,
                       kvp_stream_t stream) {
  using namespace kvp;
  kvp_pool_desc d;
  if (kvp_pool_get_desc(pool, &d) != KVP_OK) return KVP_E_INVAL;
  Geometry geo;
  const kvp_status st = prefill_geometry(d, num_seqs, num_q_heads, max_blocks, max_q_len,
                                         max_context_len, &geo);
  if (st != KVP_OK) return st;
  if (!std::isfinite(scale)) return KVP_E_INVAL;
  if (num_seqs == 0 || max_q_len == 0) return KVP_OK;
  if (!q || !q_start || !k_pool || !v_pool || !block_tables || !context_lens || !out)
    return KVP_E_INVAL;
  if (geo.quant != (k_meta != nullptr) || geo.quant != (v_meta != nullptr)) return KVP_E_INVAL;
  if (order && order_len > 0x7fffffff) return KVP_E_UNSUPPORTED;
  const int64_t grid_len = order ? order_len : geo.wgs;
  if (grid_len == 0) return KVP_OK;
  PrefillArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.q_start = q_start;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_meta = static_cast<const uint16_t*>(k_meta);
  a.v_meta = static_cast<const uint16_t*>(v_meta);
  a.bt = block_tables;
  a.ctx_lens = context_lens;
  a.out = static_cast<uint16_t*>(out);
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks;
  a.num_kv_heads = d.num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.group = geo.g;
  a.num_pages = d.num_pages;
  a.tiles = int32_t(geo.tiles);
  a.ctx_cap = max_context_len;
  a.scale_log2 = scale * kLog2e;
  a.order = order;
  a.units = int32_t(geo.wgs);
  const dim3 grid(static_cast<unsigned>(grid_len));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  const int P = d.page_size, D = d.head_dim;
  switch (d.dtype) {
    case KVP_BF16: e = launch_prefill_fmt<kBF16>(a, P, D, geo.nt, geo.split, grid, s); break;
    case KVP_INT8: e = launch_prefill_fmt<kI8>(a, P, D, geo.nt, geo.split, grid, s); break;
    case KVP_INT4: e = launch_prefill_fmt<kI4>(a, P, D, geo.nt, geo.split, grid, s); break;
    default: e = launch_prefill_fmt<kFP8>(a, P, D, geo.nt, geo.split, grid, s); break;
  }
  return e == hipSuccess ? KVP_OK : KVP_E_HIP;
}

}  // namespace

extern "C" kvp_status kvp_paged_attention_prefill(
    const kvp_pool* pool, const void* q, const int32_t* q_start, const void* k_pool,
    const void* v_pool, const void* k_meta, const void* v_meta, const int32_t* block_tables,
    int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
    int32_t max_q_len, int32_t max_context_len, float scale, void* out, kvp_stream_t stream) {
  return prefill_run(pool, q, q_start, k_pool, v_pool, k_meta, v_meta, block_tables, max_blocks,
                     context_lens, num_seqs, num_q_heads, max_q_len, max_context_len, scale,
                     nullptr, 0, out, stream);
}

extern "C" kvp_status kvp_prefill_schedule_bound(const kvp_pool* pool, int32_t num_seqs,
                                                 int32_t num_q_heads, int32_t max_blocks,
                                                 int32_t max_q_len, int32_t max_context_len,
                                                 int64_t* max_entries) {
  kvp_pool_desc d;
  if (!max_entries || kvp_pool_get_desc(pool, &d) != KVP_OK) return KVP_E_INVAL;
  Geometry geo;
  const kvp_status st = prefill_geometry(d, num_seqs, num_q_heads, max_blocks, max_q_len,
                                         max_context_len, &geo);
  if (st != KVP_OK) return st;
  *max_entries = 8 * geo.wgs;
  return KVP_OK;
}

// Longest-first order of the natural grid's units (see the header): a unit's
// cost is the number of 64-key blocks its last row sees, plus one; items go to
// the XCD with the least cost so far (costliest item first), or, when that
// leaves one XCD more than 1.2x the mean, the units do; each XCD runs its
// units costliest first.
extern "C" kvp_status kvp_prefill_schedule(const kvp_pool* pool, const int32_t* q_start,
                                           const int32_t* context_lens, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t max_blocks,
                                           int32_t max_q_len, int32_t max_context_len,
                                           int32_t* sched, int64_t capacity, int64_t* entries) {
  kvp_pool_desc d;
  if (!entries || kvp_pool_get_desc(pool, &d) != KVP_OK) return KVP_E_INVAL;
  Geometry geo;
  const kvp_status st = prefill_geometry(d, num_seqs, num_q_heads, max_blocks, max_q_len,
                                         max_context_len, &geo);
  if (st != KVP_OK) return st;
  if (num_seqs > 0 && (!q_start || !context_lens)) return KVP_E_INVAL;
  if (capacity < 0 || (capacity > 0 && !sched)) return KVP_E_INVAL;
  if (num_seqs > 0 && q_start[0] != 0) return KVP_E_INVAL;
  for (int32_t b = 0; b < num_seqs; ++b)
    if (q_start[b + 1] < q_start[b] || context_lens[b] < 0) return KVP_E_INVAL;
  const int H = d.num_kv_heads, g = geo.g;
  const int64_t per_group = 8 * geo.tiles;
  std::vector<int64_t> cost(size_t(geo.wgs), 0), item_cost(size_t(geo.items), 0);
  for (int64_t u = 0; u < geo.wgs; ++u) {
    const int64_t grp = u / per_group, within = u - grp * per_group;
    const int64_t tile = within >> 3, item = grp * 8 + (within & 7);
    if (item >= geo.items) continue;
    const int64_t b = item / H;
    const int64_t qlen = int64_t(q_start[b + 1]) - q_start[b];
    const int64_t rows = qlen * g;
    const int64_t row0 = geo.split ? 0 : tile * geo.rows_wg;
    if (qlen <= 0 || row0 >= rows) continue;   // the kernel does nothing there
    const int64_t ctx = std::min<int64_t>(context_lens[b], max_context_len);
    const int64_t row_last = std::min(row0 + geo.rows_wg, rows) - 1;
    const int64_t pos_last = std::min(ctx - qlen + row_last / g, ctx - 1);
    cost[size_t(u)] = (pos_last >= 0 ? pos_last / 64 + 1 : 0) + 1;
    item_cost[size_t(item)] += cost[size_t(u)];
  }
  std::vector<int64_t> items(size_t(geo.items));
  for (int64_t i = 0; i < geo.items; ++i) items[size_t(i)] = i;
  std::stable_sort(items.begin(), items.end(), [&](int64_t x, int64_t y) {
    return item_cost[size_t(x)] > item_cost[size_t(y)];
  });
  auto least_loaded = [](const int64_t* load) {
    int x = 0;
    for (int k = 1; k < 8; ++k)
      if (load[k] < load[x]) x = k;
    return x;
  };
  std::vector<int> xcd_of(size_t(geo.items), 0);
  int64_t load[8] = {0, 0, 0, 0, 0, 0, 0, 0}, total = 0;
  for (int64_t it : items) {
    const int x = least_loaded(load);
    xcd_of[size_t(it)] = x;
    load[x] += item_cost[size_t(it)];
    total += item_cost[size_t(it)];
  }
  // Too few (or too uneven) items to share out whole: one XCD would carry
  // more than 1.2x the mean.  Then the units themselves are shared out,
  // costliest first, and an item's tiles no longer share one L2.
  const bool by_unit = 10 * 8 * *std::max_element(load, load + 8) > 12 * total;
  std::vector<int64_t> lists[8];
  if (by_unit) {
    std::vector<int64_t> order_u;
    for (int64_t u = 0; u < geo.wgs; ++u)
      if (cost[size_t(u)] > 0) order_u.push_back(u);
    std::stable_sort(order_u.begin(), order_u.end(),
                     [&](int64_t x, int64_t y) { return cost[size_t(x)] > cost[size_t(y)]; });
    std::fill(load, load + 8, 0);
    for (int64_t u : order_u) {
      const int x = least_loaded(load);
      lists[x].push_back(u);
      load[x] += cost[size_t(u)];
    }
  } else {
    for (int64_t u = 0; u < geo.wgs; ++u) {
      if (cost[size_t(u)] == 0) continue;
      const int64_t grp = u / per_group, within = u - grp * per_group;
      lists[xcd_of[size_t(grp * 8 + (within & 7))]].push_back(u);
    }
  }
  size_t longest = 0;
  for (auto& l : lists) {
    std::stable_sort(l.begin(), l.end(),
                     [&](int64_t x, int64_t y) { return cost[size_t(x)] > cost[size_t(y)]; });
    longest = std::max(longest, l.size());
  }
  const int64_t n = 8 * int64_t(longest);
  *entries = n;
  if (n > capacity) return KVP_E_INVAL;
  for (int64_t r = 0; r < int64_t(longest); ++r)
    for (int x = 0; x < 8; ++x)
      sched[8 * r + x] = r < int64_t(lists[x].size()) ? int32_t(lists[x][size_t(r)]) : -1;
  return KVP_OK;
}

extern "C" kvp_status kvp_paged_attention_prefill_scheduled(
    const kvp_pool* pool, const void* q, const int32_t* q_start, const void* k_pool,
    const void* v_pool, const void* k_meta, const void* v_meta, const int32_t* block_tables,
    int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
    int32_t max_q_len, int32_t max_context_len, float scale, const int32_t* sched,
    int64_t entries, void* out, kvp_stream_t stream) {
  if (entries < 0 || (entries > 0 && !sched)) return KVP_E_INVAL;
  if (entries == 0) return KVP_OK;
  return prefill_run(pool, q, q_start, k_pool, v_pool, k_meta, v_meta, block_tables, max_blocks,
                     context_lens, num_seqs, num_q_heads, max_q_len, max_context_len, scale, sched,
                     entries, out, stream);
}
