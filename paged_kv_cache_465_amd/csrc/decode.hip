// Paged decode attention for gfx950: host side of the C ABI (planning,
// argument checks, launches).  The kernels are in decode_kernels.h; the
// instances of each (KV format, plan) are compiled in a file of their own,
// decode_<format>_split.hip and decode_<format>_sched.hip.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "decode_kernels.h"

namespace kvp {

// Instantiated in the per-format files.
#define KVP_DECODE_FMT_EXTERN(F)                                                    \
  extern template hipError_t launch_decode_fmt<F, false>(const DecodeArgs&, int, int, bool, \
                                                         int, dim3, dim3, size_t,        \
                                                         hipStream_t);                   \
  extern template hipError_t launch_decode_fmt<F, true>(const DecodeArgs&, int, int, bool,  \
                                                        int, dim3, dim3, size_t, hipStream_t);
KVP_DECODE_FMT_EXTERN(kBF16)
KVP_DECODE_FMT_EXTERN(kI8)
KVP_DECODE_FMT_EXTERN(kI4)
KVP_DECODE_FMT_EXTERN(kFP8)
#undef KVP_DECODE_FMT_EXTERN

int cu_count_current_device() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  if (dev < 64) cache[dev] = n;
  return n;
}

template <bool SCHED>
hipError_t launch_decode_dtype(const DecodeArgs& a, int dtype, int P, int D, bool mfma, int g,
                               dim3 grid, dim3 block, size_t lds, hipStream_t s) {
  switch (dtype) {
    case KVP_BF16: return launch_decode_fmt<kBF16, SCHED>(a, P, D, mfma, g, grid, block, lds, s);
    case KVP_INT8: return launch_decode_fmt<kI8, SCHED>(a, P, D, mfma, g, grid, block, lds, s);
    case KVP_INT4: return launch_decode_fmt<kI4, SCHED>(a, P, D, mfma, g, grid, block, lds, s);
    case KVP_FP8: return launch_decode_fmt<kFP8, SCHED>(a, P, D, mfma, g, grid, block, lds, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvp

namespace {

size_t partials_o_bytes(size_t parts, int D) {
  return (parts * size_t(D) * sizeof(float) + 255) & ~size_t(255);
}

size_t partials_bytes(size_t parts, int D) {
  return partials_o_bytes(parts, D) + parts * 2 * sizeof(float);
}

hipError_t launch_merge(const float* part_o, const float* part_ml, uint16_t* out, int rows, int S,
                        int D, hipStream_t s) {
  kvp::discard_stale_error();
  const dim3 mg(static_cast<unsigned>((rows + 3) / 4));
  if (D == 128)
    hipLaunchKernelGGL((kvp::merge_kernel<128>), mg, dim3(256), 0, s, part_o, part_ml, out, rows, S);
  else
    hipLaunchKernelGGL((kvp::merge_kernel<64>), mg, dim3(256), 0, s, part_o, part_ml, out, rows, S);
  return hipGetLastError();
}

// Validate the decode arguments and fill the plan.  partials_only forces the
// split kernel to write (o, m, l) partials even for one split.
// Tokens the planner sizes splits for: with a window, a sequence streams at
// most ceil(sink/P) + ceil(window/P) + 1 pages.
int32_t planned_context(int32_t max_context_len, int32_t page_size, int32_t sink_tokens,
                        int32_t window_tokens) {
  if (window_tokens <= 0) return max_context_len;
  const int64_t blocks = (int64_t(sink_tokens) + page_size - 1) / page_size +
                         (int64_t(window_tokens) + page_size - 1) / page_size + 1;
  return int32_t(std::min<int64_t>(max_context_len, blocks * page_size));
}

kvp_status prepare_decode(const kvp_pool* pool, const void* q, const void* k_pool,
                          const void* v_pool, const void* k_meta, const void* v_meta,
                          const int32_t* block_tables, int32_t max_blocks,
                          const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                          int32_t max_context_len, float scale, int32_t num_splits_req,
                          int32_t sink_tokens, int32_t window_tokens,
                          kvp_pool_desc* d, kvp_decode_plan_t* plan, bool* empty) {
  *empty = false;
  if (kvp_pool_get_desc(pool, d) != KVP_OK) return KVP_E_INVAL;
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks <= 0) return KVP_E_INVAL;
  if (num_q_heads % d->num_kv_heads) return KVP_E_INVAL;
  if (int64_t(max_blocks) * d->page_size > 0x7fffffff) return KVP_E_INVAL;
  if (max_context_len < 0 || int64_t(max_context_len) > int64_t(max_blocks) * d->page_size)
    return KVP_E_INVAL;
  if (!std::isfinite(scale)) return KVP_E_INVAL;
  if (sink_tokens < 0 || window_tokens < 0) return KVP_E_INVAL;
  if (num_seqs == 0) {
    *empty = true;
    return KVP_OK;
  }
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens) return KVP_E_INVAL;
  const bool quant = d->dtype != KVP_BF16;
  if (quant != (k_meta != nullptr) || quant != (v_meta != nullptr)) return KVP_E_INVAL;
  const int cus = kvp::cu_count_current_device();
  if (cus <= 0) return KVP_E_HIP;
  const kvp_status st = kvp_decode_plan(
      d, num_seqs, num_q_heads,
      planned_context(max_context_len, d->page_size, sink_tokens, window_tokens),
      num_splits_req, cus, plan);
  if (st != KVP_OK) return st;
  if (int64_t(num_seqs) * d->num_kv_heads * plan->num_splits > 0x7fffffff)
    return KVP_E_UNSUPPORTED;
  return KVP_OK;
}

kvp_status launch_split_kernel(const kvp_pool_desc& d, const kvp_decode_plan_t& plan,
                               const void* q, const void* k_pool, const void* v_pool,
                               const void* k_meta, const void* v_meta,
                               const int32_t* block_tables, int32_t max_blocks,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t max_context_len, float scale,
                               int32_t sink_tokens, int32_t window_tokens,
                               void* out, float* part_o, float* part_ml, hipStream_t s,
                               const kvp_schedule_info* sched_info = nullptr,
                               const int32_t* sched = nullptr) {
  using namespace kvp;
  const int g = num_q_heads / d.num_kv_heads;
  DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_meta = static_cast<const uint16_t*>(k_meta);
  a.v_meta = static_cast<const uint16_t*>(v_meta);
  a.bt = block_tables;
  a.ctx_lens = context_lens;
  a.out = static_cast<uint16_t*>(out);
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks;
  a.num_kv_heads = d.num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.group = g;
  a.num_pages = d.num_pages;
  a.num_splits = plan.num_splits;
  a.pages_per_split = plan.pages_per_split;
  a.ctx_cap = max_context_len;
  a.sink_tokens = sink_tokens;
  a.window_tokens = window_tokens;
  a.write_partials = part_o != nullptr;
  a.scale_log2 = scale * kLog2e;
  a.sched = sched;
  a.items_off = sched ? sched_info->items_offset : 0;
  a.num_items = sched ? sched_info->num_items : 0;
  // partial slots exist only with a partials buffer: without one, an item
  // naming a slot is skipped instead of writing through a null pointer
  a.num_slots = sched && part_o ? sched_info->num_slots : 0;
  a.num_bins = sched ? sched_info->num_bins : 0;

  const int W = plan.waves_per_group;
  const int HP = plan.use_mfma ? ((g + 15) / 16) * 16 : g;
  size_t lds = size_t(W) * (size_t(g) * d.head_dim + 2 * HP) * sizeof(float);
  if (!plan.use_mfma) lds += size_t(W) * g * d.page_size * sizeof(float);
  // balanced schedule: a bin is a wavefront on the matrix-core path, a
  // workgroup on the vector path
  const int64_t wgs =
      !sched ? int64_t(num_seqs) * d.num_kv_heads * plan.num_splits
             : (plan.use_mfma ? (int64_t(sched_info->num_bins) + W - 1) / W
                              : int64_t(sched_info->num_bins));
  const dim3 grid(static_cast<unsigned>(wgs)), block(static_cast<unsigned>(W * 64));
  const int P = d.page_size, D = d.head_dim;
  const bool mf = plan.use_mfma;
  const hipError_t e =
      sched ? launch_decode_dtype<true>(a, d.dtype, P, D, mf, g, grid, block, lds, s)
            : launch_decode_dtype<false>(a, d.dtype, P, D, mf, g, grid, block, lds, s);
  return e == hipSuccess ? KVP_OK : KVP_E_HIP;
}

}  // namespace

extern "C" kvp_status kvp_decode_workspace_bytes(const kvp_pool* pool, int32_t num_seqs,
                                                 int32_t num_q_heads, int32_t max_context_len,
                                                 int32_t num_splits_req, size_t* bytes) {
  kvp_pool_desc d;
  if (!bytes || kvp_pool_get_desc(pool, &d) != KVP_OK) return KVP_E_INVAL;
  const int cus = kvp::cu_count_current_device();
  if (cus <= 0) return KVP_E_HIP;
  kvp_decode_plan_t plan;
  const kvp_status st =
      kvp_decode_plan(&d, num_seqs, num_q_heads, max_context_len, num_splits_req, cus, &plan);
  if (st != KVP_OK) return st;
  *bytes = plan.workspace_bytes;
  return KVP_OK;
}

namespace {

kvp_status decode_full(const kvp_pool* pool, const void* q, const void* k_pool, const void* v_pool,
                       const void* k_meta, const void* v_meta, const int32_t* block_tables,
                       int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs,
                       int32_t num_q_heads, int32_t max_context_len, float scale,
                       int32_t sink_tokens, int32_t window_tokens, void* out,
                       int32_t num_splits_req, void* workspace, size_t workspace_bytes,
                       kvp_stream_t stream) {
  kvp_pool_desc d;
  kvp_decode_plan_t plan;
  bool empty;
  kvp_status st = prepare_decode(pool, q, k_pool, v_pool, k_meta, v_meta, block_tables,
                                 max_blocks, context_lens, num_seqs, num_q_heads,
                                 max_context_len, scale, num_splits_req, sink_tokens,
                                 window_tokens, &d, &plan, &empty);
  if (st != KVP_OK || empty) return st;
  if (!out) return KVP_E_INVAL;
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return KVP_E_INVAL;
  const size_t parts = size_t(num_seqs) * num_q_heads * plan.num_splits;
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (plan.num_splits > 1) {
    part_o = static_cast<float*>(workspace);
    part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       partials_o_bytes(parts, d.head_dim));
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = launch_split_kernel(d, plan, q, k_pool, v_pool, k_meta, v_meta, block_tables, max_blocks,
                           context_lens, num_seqs, num_q_heads, max_context_len, scale,
                           sink_tokens, window_tokens, out, part_o, part_ml, s);
  if (st != KVP_OK) return st;
  if (plan.num_splits > 1 &&
      launch_merge(part_o, part_ml, static_cast<uint16_t*>(out), num_seqs * num_q_heads,
                   plan.num_splits, d.head_dim, s) != hipSuccess)
    return KVP_E_HIP;
  return KVP_OK;
}

}  // namespace

extern "C" kvp_status kvp_paged_attention_decode(
    const kvp_pool* pool, const void* q, const void* k_pool, const void* v_pool,
    const void* k_meta, const void* v_meta, const int32_t* block_tables, int32_t max_blocks,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
    float scale, void* out, int32_t num_splits_req, void* workspace, size_t workspace_bytes,
    kvp_stream_t stream) {
  return decode_full(pool, q, k_pool, v_pool, k_meta, v_meta, block_tables, max_blocks,
                     context_lens, num_seqs, num_q_heads, max_context_len, scale, 0, 0, out,
                     num_splits_req, workspace, workspace_bytes, stream);
}

// ---- Decode without a caller workspace --------------------------------------
// For callers that cannot allocate device memory: the split partials live in
// one file-scope device array per GPU, held until the process ends.  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): the device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// used.  Every partial a call reads was written earlier in the same call
// (empty splits write m = -inf, l = 0), so nothing needs clearing.
static __device__ __align__(256) unsigned char scratch[KVP_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

kvp_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return KVP_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      kvp::discard_stale_error();
      return KVP_E_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVP_OK;
}

}  // namespace

extern "C" kvp_status kvp_paged_attention_decode_noalloc(
    const kvp_pool* pool, const void* q, const void* k_pool, const void* v_pool,
    const void* k_meta, const void* v_meta, const int32_t* block_tables, int32_t max_blocks,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
    float scale, void* out, int32_t num_splits_req, kvp_stream_t stream) {
  kvp_pool_desc d;
  kvp_decode_plan_t plan;
  bool empty;
  const kvp_status st = prepare_decode(pool, q, k_pool, v_pool, k_meta, v_meta, block_tables,
                                       max_blocks, context_lens, num_seqs, num_q_heads,
                                       max_context_len, scale, num_splits_req, 0, 0, &d, &plan,
                                       &empty);
  if (st != KVP_OK || empty) return st;
  if (plan.workspace_bytes > KVP_DECODE_SCRATCH_BYTES) return KVP_E_SCRATCH;
  void* ws = nullptr;
  if (plan.workspace_bytes > 0) {
    const kvp_status sst = scratch_of_current_device(&ws);
    if (sst != KVP_OK) return sst;
  }
  return decode_full(pool, q, k_pool, v_pool, k_meta, v_meta, block_tables, max_blocks,
                     context_lens, num_seqs, num_q_heads, max_context_len, scale, 0, 0, out,
                     num_splits_req, ws, KVP_DECODE_SCRATCH_BYTES, stream);
}

extern "C" kvp_status kvp_decode_window_workspace_bytes(const kvp_pool* pool, int32_t num_seqs,
                                                        int32_t num_q_heads,
                                                        int32_t max_context_len,
                                                        int32_t sink_tokens,
                                                        int32_t window_tokens,
                                                        int32_t num_splits_req, size_t* bytes) {
  kvp_pool_desc d;
  if (!bytes || kvp_pool_get_desc(pool, &d) != KVP_OK) return KVP_E_INVAL;
  if (sink_tokens < 0 || window_tokens < 0 || max_context_len < 0) return KVP_E_INVAL;
  return kvp_decode_workspace_bytes(
      pool, num_seqs, num_q_heads,
      planned_context(max_context_len, d.page_size, sink_tokens, window_tokens), num_splits_req,
      bytes);
}

extern "C" kvp_status kvp_paged_attention_decode_window(
    const kvp_pool* pool, const void* q, const void* k_pool, const void* v_pool,
    const void* k_meta, const void* v_meta, const int32_t* block_tables, int32_t max_blocks,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
    float scale, int32_t sink_tokens, int32_t window_tokens, void* out, int32_t num_splits_req,
    void* workspace, size_t workspace_bytes, kvp_stream_t stream) {
  return decode_full(pool, q, k_pool, v_pool, k_meta, v_meta, block_tables, max_blocks,
                     context_lens, num_seqs, num_q_heads, max_context_len, scale, sink_tokens,
                     window_tokens, out, num_splits_req, workspace, workspace_bytes, stream);
}

extern "C" kvp_status kvp_decode_partials_bytes(const kvp_pool* pool, int32_t num_seqs,
                                                int32_t num_q_heads, int32_t max_context_len,
                                                int32_t num_splits_req, int32_t* num_splits,
                                                size_t* bytes) {
  kvp_pool_desc d;
  if (!bytes || kvp_pool_get_desc(pool, &d) != KVP_OK) return KVP_E_INVAL;
  const int cus = kvp::cu_count_current_device();
  if (cus <= 0) return KVP_E_HIP;
  kvp_decode_plan_t plan;
  const kvp_status st =
      kvp_decode_plan(&d, num_seqs, num_q_heads, max_context_len, num_splits_req, cus, &plan);
  if (st != KVP_OK) return st;
  if (num_splits) *num_splits = plan.num_splits;
  *bytes = partials_bytes(size_t(num_seqs) * num_q_heads * plan.num_splits, d.head_dim);
  return KVP_OK;
}

extern "C" kvp_status kvp_paged_attention_decode_partials(
    const kvp_pool* pool, const void* q, const void* k_pool, const void* v_pool,
    const void* k_meta, const void* v_meta, const int32_t* block_tables, int32_t max_blocks,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
    float scale, int32_t num_splits_req, void* partials, size_t partials_bytes_avail,
    int32_t* num_splits, kvp_stream_t stream) {
  kvp_pool_desc d;
  kvp_decode_plan_t plan;
  bool empty;
  kvp_status st = prepare_decode(pool, q, k_pool, v_pool, k_meta, v_meta, block_tables,
                                 max_blocks, context_lens, num_seqs, num_q_heads,
                                 max_context_len, scale, num_splits_req, 0, 0, &d, &plan, &empty);
  if (st != KVP_OK) return st;
  if (empty) {
    if (num_splits) *num_splits = 0;
    return KVP_OK;
  }
  const size_t parts = size_t(num_seqs) * num_q_heads * plan.num_splits;
  if (!partials || partials_bytes_avail < partials_bytes(parts, d.head_dim)) return KVP_E_INVAL;
  float* part_o = static_cast<float*>(partials);
  float* part_ml = reinterpret_cast<float*>(static_cast<char*>(partials) +
                                            partials_o_bytes(parts, d.head_dim));
  st = launch_split_kernel(d, plan, q, k_pool, v_pool, k_meta, v_meta, block_tables, max_blocks,
                           context_lens, num_seqs, num_q_heads, max_context_len, scale, 0, 0,
                           nullptr, part_o, part_ml, reinterpret_cast<hipStream_t>(stream));
  if (st == KVP_OK && num_splits) *num_splits = plan.num_splits;
  return st;
}

extern "C" kvp_status kvp_lse_merge(const void* partials, int32_t rows, int32_t num_splits,
                                    int32_t head_dim, void* out, kvp_stream_t stream) {
  if (rows < 0 || num_splits <= 0 || (head_dim != 64 && head_dim != 128)) return KVP_E_INVAL;
  if (rows == 0) return KVP_OK;
  if (!partials || !out) return KVP_E_INVAL;
  const size_t parts = size_t(rows) * num_splits;
  const float* part_o = static_cast<const float*>(partials);
  const float* part_ml = reinterpret_cast<const float*>(static_cast<const char*>(partials) +
                                                        partials_o_bytes(parts, head_dim));
  return launch_merge(part_o, part_ml, static_cast<uint16_t*>(out), rows, num_splits, head_dim,
                      reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? KVP_OK
             : KVP_E_HIP;
}

extern "C" kvp_status kvp_decode_schedule_bins(const kvp_pool* pool, int32_t num_q_heads,
                                               int32_t* max_bins) {
  kvp_pool_desc d;
  if (!max_bins || kvp_pool_get_desc(pool, &d) != KVP_OK || num_q_heads <= 0 ||
      num_q_heads % d.num_kv_heads)
    return KVP_E_INVAL;
  const int cus = kvp::cu_count_current_device();
  if (cus <= 0) return KVP_E_HIP;
  // the planner's choice of kernel family for this group size
  kvp_decode_plan_t plan;
  if (kvp_decode_plan(&d, 1, num_q_heads, d.page_size, 0, cus, &plan) != KVP_OK)
    return KVP_E_INVAL;
  // wavefronts per SIMD of the stream kernel: quantized pools with one head
  // tile (g <= 16) run two (INT4: three)
  const int g = num_q_heads / d.num_kv_heads;
  const int waves =
      plan.use_mfma && d.dtype != KVP_BF16 && g <= 16 ? (d.dtype == KVP_INT4 ? 3 : 2) : 1;
  *max_bins = 4 * waves * cus;
  return KVP_OK;
}

extern "C" kvp_status kvp_paged_attention_decode_scheduled(
    const kvp_pool* pool, const void* q, const void* k_pool, const void* v_pool,
    const void* k_meta, const void* v_meta, const int32_t* block_tables, int32_t max_blocks,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
    float scale, const int32_t* sched, const kvp_schedule_info* info, void* out,
    void* workspace, size_t workspace_bytes, kvp_stream_t stream) {
  if (!info) return KVP_E_INVAL;
  // the schedule's header first (host only): a schedule that cuts pairs has
  // partial slots and merge entries, and one that cuts none has neither, so
  // an info with slots but no merge entries (or the reverse) is not one
  // kvp_decode_schedule built; refusing it keeps partial writes behind a
  // workspace the call has checked
  const int64_t bins = info->num_bins, items = info->num_items;
  if (bins < 1 || items < 0 || info->num_merge < 0 || info->num_slots < 0 ||
      (info->num_merge == 0) != (info->num_slots == 0) ||
      info->items_offset < 8 + bins + 1 ||
      int64_t(info->merge_offset) != info->items_offset + 8 * items)
    return KVP_E_INVAL;
  kvp_pool_desc d;
  kvp_decode_plan_t plan;
  bool empty;
  kvp_status st = prepare_decode(pool, q, k_pool, v_pool, k_meta, v_meta, block_tables,
                                 max_blocks, context_lens, num_seqs, num_q_heads,
                                 max_context_len, scale, 1, info->sink_tokens,
                                 info->window_tokens, &d, &plan, &empty);
  if (st != KVP_OK || empty) return st;
  if (!out || !sched) return KVP_E_INVAL;
  const int g = num_q_heads / d.num_kv_heads;
  const size_t slots = size_t(info->num_slots);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (info->num_merge > 0) {
    const size_t o_bytes = (slots * g * d.head_dim * sizeof(float) + 255) & ~size_t(255);
    if (!workspace || workspace_bytes < o_bytes + slots * g * 2 * sizeof(float))
      return KVP_E_INVAL;
    part_o = static_cast<float*>(workspace);
    part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = launch_split_kernel(d, plan, q, k_pool, v_pool, k_meta, v_meta, block_tables, max_blocks,
                           context_lens, num_seqs, num_q_heads, max_context_len, scale,
                           info->sink_tokens, info->window_tokens, out, part_o, part_ml, s, info,
                           sched);
  if (st != KVP_OK || info->num_merge == 0) return st;
  const int rows = info->num_merge * g;
  const dim3 mg(static_cast<unsigned>((rows + 3) / 4));
  const int32_t* entries = sched + info->merge_offset;
  kvp::discard_stale_error();
  uint16_t* o16 = static_cast<uint16_t*>(out);
  if (d.head_dim == 128)
    hipLaunchKernelGGL((kvp::merge_sched_kernel<128>), mg, dim3(256), 0, s, part_o, part_ml,
                       entries, o16, rows, g, num_q_heads, num_seqs, info->num_slots);
  else
    hipLaunchKernelGGL((kvp::merge_sched_kernel<64>), mg, dim3(256), 0, s, part_o, part_ml,
                       entries, o16, rows, g, num_q_heads, num_seqs, info->num_slots);
  return hipGetLastError() == hipSuccess ? KVP_OK : KVP_E_HIP;
}
