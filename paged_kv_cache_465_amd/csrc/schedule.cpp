// Balanced decode schedule from host-side context lengths.
//
// "KV-Cache Optimization Techniques", section "PagedAttention": a sequence's
// K/V live in its pages, so the work of one decode step is the list of
// (sequence, KV head, page) triples; with ragged lengths an even share of
// that list per compute unit, rather than an even share per sequence, is what
// keeps every unit streaming until the end.
//
// The (sequence, KV head) pairs are laid end to end (head fastest), each
// contributing its streamed block count (the sink + window selection of the
// "Token Eviction Strategies" section, eq. 5, shrinks it).  Bin k of
// num_bins covers blocks [k*T/num_bins, (k+1)*T/num_bins) of that list.
// The pieces a bin covers become its items, processed one after another by
// one wavefront (matrix-core path) or workgroup (vector path).  A pair
// inside one bin writes its output directly; a pair
// cut by bin boundaries writes one partial per piece, and a merge entry names
// its consecutive partial slots.
//
// Plain C++17 with no HIP dependency.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "kvp.h"

namespace {

constexpr int32_t kHeaderWords = 8;
constexpr int32_t kItemWords = 8;
constexpr int32_t kMergeWords = 4;
constexpr int64_t kMinBinBlocks = 8;  // at least two blocks per wavefront of a bin

int64_t align8(int64_t x) { return (x + 7) & ~int64_t(7); }

// Blocks a sequence of n tokens streams: all ceil(n/P), or with sinks and a
// window (sink + window < n) the sink blocks and the window's blocks.
int64_t streamed_blocks(int64_t n, int32_t P, int32_t sink, int32_t window) {
  const int64_t nblk = (n + P - 1) / P;
  if (window <= 0 || int64_t(sink) + window >= n) return nblk;
  const int64_t sink_blk = (int64_t(sink) + P - 1) / P;
  const int64_t win_first = std::max((n - window) / P, sink_blk);
  return sink_blk + (nblk - win_first);
}

struct Sizes {
  int64_t max_bins, max_items, max_merge, max_slots, words;
};

Sizes bounds(int64_t pairs, int32_t max_bins) {
  Sizes z;
  z.max_bins = std::max<int64_t>(1, max_bins);
  z.max_items = pairs + z.max_bins;
  z.max_merge = z.max_bins;
  z.max_slots = 2 * z.max_bins;
  z.words = align8(kHeaderWords + z.max_bins + 1) + z.max_items * kItemWords +
            z.max_merge * kMergeWords;
  return z;
}

size_t partial_bytes(int64_t slots, int32_t g, int32_t D) {
  size_t o = size_t(slots) * g * D * sizeof(float);
  o = (o + 255) & ~size_t(255);
  return o + size_t(slots) * g * 2 * sizeof(float);
}

}  // namespace

extern "C" {

kvp_status kvp_decode_schedule_bounds(const kvp_pool* pool, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_bins,
                                      size_t* sched_bytes, size_t* workspace_bytes) {
  kvp_pool_desc d;
  if (kvp_pool_get_desc(pool, &d) != KVP_OK || num_seqs < 0 || num_q_heads <= 0 ||
      max_bins <= 0 || !sched_bytes || !workspace_bytes)
    return KVP_E_INVAL;
  if (num_q_heads % d.num_kv_heads) return KVP_E_INVAL;
  const Sizes z = bounds(int64_t(num_seqs) * d.num_kv_heads, max_bins);
  if (z.words > 0x7fffffff) return KVP_E_UNSUPPORTED;
  *sched_bytes = size_t(z.words) * sizeof(int32_t);
  *workspace_bytes = partial_bytes(z.max_slots, num_q_heads / d.num_kv_heads, d.head_dim);
  return KVP_OK;
}

kvp_status kvp_decode_schedule(const kvp_pool* pool, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks,
                               int32_t sink_tokens, int32_t window_tokens, int32_t max_bins,
                               int32_t* sched, size_t sched_bytes, kvp_schedule_info* info) {
  kvp_pool_desc d;
  if (kvp_pool_get_desc(pool, &d) != KVP_OK || num_seqs < 0 || num_q_heads <= 0 ||
      max_blocks <= 0 || max_bins <= 0 || sink_tokens < 0 || window_tokens < 0 || !info ||
      !sched || (num_seqs > 0 && !context_lens))
    return KVP_E_INVAL;
  if (num_q_heads % d.num_kv_heads) return KVP_E_INVAL;
  const int32_t P = d.page_size, H = d.num_kv_heads;
  const int64_t pairs = int64_t(num_seqs) * H;
  const Sizes z = bounds(pairs, max_bins);
  if (z.words > 0x7fffffff) return KVP_E_UNSUPPORTED;
  if (sched_bytes < size_t(z.words) * sizeof(int32_t)) return KVP_E_INVAL;

  std::vector<int64_t> nv(static_cast<size_t>(num_seqs));
  int64_t per_head = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t n = context_lens[b];
    if (n < 0 || n > int64_t(max_blocks) * P) return KVP_E_INVAL;
    nv[b] = streamed_blocks(n, P, sink_tokens, window_tokens);
    per_head += nv[b];
  }
  const int64_t T = per_head * H;
  const int64_t bins =
      std::max<int64_t>(1, std::min<int64_t>(z.max_bins, (T + kMinBinBlocks - 1) / kMinBinBlocks));
  auto bin_begin = [&](int64_t k) { return k * T / bins; };  // exact integer cut

  int32_t* bin_start = sched + kHeaderWords;
  const int64_t items_off = align8(kHeaderWords + bins + 1);
  int32_t* items = sched + items_off;
  int64_t n_items = 0, n_slots = 0, n_merge = 0;
  std::vector<int32_t> merge;  // seq, head, first slot, count

  // Walk the pairs in order; bin k is filled while its range overlaps them.
  int64_t k = 0, off = 0;
  bin_start[0] = 0;
  for (int64_t p = 0; p < pairs; ++p) {
    const int32_t b = int32_t(p / H), h = int32_t(p % H);
    const int64_t len = nv[size_t(b)];
    // move to the bin whose range holds this pair's start (no bin is empty
    // when T > 0; empty pairs at the very end fall into the last bin)
    while (k + 1 < bins && bin_begin(k + 1) <= off) {
      ++k;
      bin_start[k] = int32_t(n_items);
    }
    if (len == 0) {
      int32_t* it = items + n_items * kItemWords;
      const int32_t rec[kItemWords] = {b, h, 0, 0, -1, 0, 0, 0};
      std::memcpy(it, rec, sizeof(rec));
      ++n_items;
      continue;
    }
    const int64_t end = off + len;
    // bins covering [off, end)
    int64_t k_last = k;
    while (k_last + 1 < bins && bin_begin(k_last + 1) < end) ++k_last;
    const bool split = k_last > k;
    const int64_t first_slot = n_slots;
    for (int64_t kk = k; kk <= k_last; ++kk) {
      if (kk > k) {
        k = kk;
        bin_start[k] = int32_t(n_items);
      }
      const int64_t lo = std::max(off, bin_begin(kk)) - off;
      const int64_t hi = std::min(end, kk + 1 < bins ? bin_begin(kk + 1) : T) - off;
      int32_t* it = items + n_items * kItemWords;
      const int32_t rec[kItemWords] = {b, h, int32_t(lo), int32_t(hi),
                                       split ? int32_t(n_slots) : -1, 0, 0, 0};
      std::memcpy(it, rec, sizeof(rec));
      ++n_items;
      if (split) ++n_slots;
    }
    if (split) {
      merge.insert(merge.end(), {b, h, int32_t(first_slot), int32_t(n_slots - first_slot)});
      ++n_merge;
    }
    off = end;
  }
  while (k + 1 < bins) {
    ++k;
    bin_start[k] = int32_t(n_items);
  }
  bin_start[bins] = int32_t(n_items);
  const int64_t merge_off = items_off + n_items * kItemWords;
  if (!merge.empty()) std::memcpy(sched + merge_off, merge.data(), merge.size() * sizeof(int32_t));
  const int32_t hdr[kHeaderWords] = {int32_t(bins), int32_t(n_items), int32_t(n_merge),
                                     int32_t(n_slots), int32_t(items_off), int32_t(merge_off),
                                     0, 0};
  std::memcpy(sched, hdr, sizeof(hdr));

  info->num_bins = int32_t(bins);
  info->num_items = int32_t(n_items);
  info->num_merge = int32_t(n_merge);
  info->num_slots = int32_t(n_slots);
  info->items_offset = int32_t(items_off);
  info->merge_offset = int32_t(merge_off);
  info->sink_tokens = sink_tokens;
  info->window_tokens = window_tokens;
  info->sched_words = int32_t(merge_off + n_merge * kMergeWords);
  info->workspace_bytes = n_slots > 0 ? partial_bytes(n_slots, num_q_heads / H, d.head_dim) : 0;
  return KVP_OK;
}

}  // extern "C"
