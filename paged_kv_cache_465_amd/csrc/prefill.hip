// Multi-query paged attention (chunked prefill, verification of drafted
// tokens): host side of the C ABI (argument checks, tiling, launches).  The
// kernel is in prefill_kernels.h; the instances of each KV format are
// compiled in a file of their own, prefill_<format>.hip.
#include <cmath>

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

extern "C" kvp_status kvp_paged_attention_prefill(
    const kvp_pool* pool, const void* q, const int32_t* q_start, const void* k_pool,
    const void* v_pool, const void* k_meta, const void* v_meta, const int32_t* block_tables,
    int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
    int32_t max_q_len, int32_t max_context_len, float scale, void* out, kvp_stream_t stream) {
  using namespace kvp;
  kvp_pool_desc d;
  if (kvp_pool_get_desc(pool, &d) != KVP_OK) return KVP_E_INVAL;
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks <= 0 || max_q_len < 0) return KVP_E_INVAL;
  if (num_q_heads % d.num_kv_heads) return KVP_E_INVAL;
  if (int64_t(max_blocks) * d.page_size > 0x7fffffff) return KVP_E_INVAL;
  if (max_context_len < 0 || int64_t(max_context_len) > int64_t(max_blocks) * d.page_size)
    return KVP_E_INVAL;
  if (!std::isfinite(scale)) return KVP_E_INVAL;
  const int g = num_q_heads / d.num_kv_heads;
  if (g > 64) return KVP_E_UNSUPPORTED;
  if (num_seqs == 0 || max_q_len == 0) return KVP_OK;
  if (!q || !q_start || !k_pool || !v_pool || !block_tables || !context_lens || !out)
    return KVP_E_INVAL;
  const bool quant = d.dtype != KVP_BF16;
  if (quant != (k_meta != nullptr) || quant != (v_meta != nullptr)) return KVP_E_INVAL;
  // rows per wavefront: 32 when the longest chunk has at least that many rows;
  // chunks whose rows fit one wavefront split the pages across the four
  const int64_t max_rows = int64_t(max_q_len) * g;
  const bool split = max_rows <= 32;
  // row-tiled mode: 128 rows per workgroup (bfloat16: the LDS-staged kernel;
  // quantized pools: 32 rows per wavefront when the longest chunk has at least
  // 128 rows, else 16)
  const int nt = split ? (max_rows > 16 ? 2 : 1) : (max_rows >= 32 * 4 || !quant ? 2 : 1);
  const int64_t rows_wg = split ? 16 * nt : (quant ? 4 * 16 * nt : 32 * kFaWaves * kFaRowTiles);
  const int64_t tiles = (max_rows + rows_wg - 1) / rows_wg;
  const int64_t items = int64_t(num_seqs) * d.num_kv_heads;
  const int64_t wgs = (items + 7) / 8 * 8 * tiles;
  if (tiles > 0x7fffffff || wgs > 0x7fffffff) return KVP_E_UNSUPPORTED;
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
  a.group = g;
  a.num_pages = d.num_pages;
  a.tiles = int32_t(tiles);
  a.ctx_cap = max_context_len;
  a.scale_log2 = scale * kLog2e;
  const dim3 grid(static_cast<unsigned>(wgs));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  const int P = d.page_size, D = d.head_dim;
  switch (d.dtype) {
    case KVP_BF16: e = launch_prefill_fmt<kBF16>(a, P, D, nt, split, grid, s); break;
    case KVP_INT8: e = launch_prefill_fmt<kI8>(a, P, D, nt, split, grid, s); break;
    case KVP_INT4: e = launch_prefill_fmt<kI4>(a, P, D, nt, split, grid, s); break;
    default: e = launch_prefill_fmt<kFP8>(a, P, D, nt, split, grid, s); break;
  }
  return e == hipSuccess ? KVP_OK : KVP_E_HIP;
}
