// kv_append: write new K/V rows into the slots their block tables name.
//
// "KV-Cache Optimization Techniques", section "PagedAttention": the page table
// maps a token's logical position to a physical page; position pos sits in
// page block_table[pos / P] at row pos % P.  INT8 pools store each (token, KV
// head) row quantized per token (section "KV-Cache Quantization", eq. 3) with
// a float16 scale and zero point, following the row contract in kvp.h.
//
// One wavefront per (token, KV head) row: each lane holds D/64 channels; the
// row's min and max come from a wavefront reduction.
#include <algorithm>

#include "device_common.h"
#include "kvp.h"

namespace kvp {

struct AppendArgs {
  void* k_pool;
  void* v_pool;
  uint16_t* k_meta;
  uint16_t* v_meta;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* seq_idx;
  const int32_t* pos;
  const int32_t* bt;
  int64_t row0;  // first (token, head) row of this launch
  int32_t n_tokens, num_seqs, max_blocks, num_pages, num_kv_heads;
};

// The row contract, one IEEE float32 operation at a time (no contraction):
// z = f16((mx+mn)*0.5), s = f16((mx-mn)/254) (1 if 0),
// code = clamp(rint_even((x - z)/s), -128, 127).
template <int E>
__device__ __forceinline__ void quantize_row(const float (&x)[E], int32_t (&code)[E],
                                             uint32_t& scale_zero) {
#pragma clang fp contract(off)
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int e = 1; e < E; ++e) {
    mn = fminf(mn, x[e]);
    mx = fmaxf(mx, x[e]);
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  float zf = (mx + mn) * 0.5f;
  // keep the float32 product: fused into one f32->f16 fma the midpoint of an
  // all -0 row would round to +0 instead of -0
  asm volatile("" : "+v"(zf));
  const _Float16 z16 = (_Float16)zf;
  const float sf = (mx - mn) / 254.0f;
  _Float16 s16 = (_Float16)sf;
  if (s16 == (_Float16)0.0f) s16 = (_Float16)1.0f;
  const float z = (float)z16, s = (float)s16;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float q = __builtin_rintf((x[e] - z) / s);
    q = fminf(fmaxf(q, -128.0f), 127.0f);
    code[e] = (int32_t)q;
  }
  scale_zero = uint32_t(__builtin_bit_cast(uint16_t, s16)) |
               (uint32_t(__builtin_bit_cast(uint16_t, z16)) << 16);
}

template <int P, int D, bool INT8>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int E = D / 64;  // channels per lane
  const int lane = threadIdx.x & 63;
  const int64_t item = a.row0 + int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int H = a.num_kv_heads;
  if (item >= int64_t(a.n_tokens) * H) return;
  const int n = int(item / H), h = int(item % H);
  const int sq = a.seq_idx[n], ps = a.pos[n];
  if (sq < 0 || sq >= a.num_seqs || ps < 0 || ps >= a.max_blocks * P) return;
  const int page = a.bt[int64_t(sq) * a.max_blocks + ps / P];
  if (page < 0 || page >= a.num_pages) return;
  const int t = ps % P;
  const int64_t tile = int64_t(page) * H + h;  // (page, head) tile index
  const int d0 = lane * E;
  const int64_t src = (int64_t(n) * H + h) * D + d0;

  uint32_t kb[E], vb[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kb[e] = a.k_new[src + e];
    vb[e] = a.v_new[src + e];
  }
  if (!INT8) {
    uint16_t* K = static_cast<uint16_t*>(a.k_pool);
    uint16_t* V = static_cast<uint16_t*>(a.v_pool);
    const int64_t krow = (tile * P + t) * D + d0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      K[krow + e] = uint16_t(kb[e]);
      V[(tile * D + d0 + e) * P + t] = uint16_t(vb[e]);
    }
    return;
  }
  int8_t* K = static_cast<int8_t*>(a.k_pool);
  int8_t* V = static_cast<int8_t*>(a.v_pool);
  float xk[E], xv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    xk[e] = bf16_to_f32(kb[e]);
    xv[e] = bf16_to_f32(vb[e]);
  }
  int32_t ck[E], cv[E];
  uint32_t mk, mv;
  quantize_row<E>(xk, ck, mk);
  quantize_row<E>(xv, cv, mv);
  const int64_t krow = (tile * P + t) * D + d0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    K[krow + e] = int8_t(ck[e]);
    V[(tile * D + d0 + e) * P + t] = int8_t(cv[e]);
  }
  if (lane == 0) {
    const int64_t m = (tile * P + t) * 2;
    *reinterpret_cast<uint32_t*>(a.k_meta + m) = mk;
    *reinterpret_cast<uint32_t*>(a.v_meta + m) = mv;
  }
}

template <int P, int D, bool INT8>
hipError_t launch_append(AppendArgs a, hipStream_t stream) {
  const int64_t rows = int64_t(a.n_tokens) * a.num_kv_heads;
  const int64_t chunk = int64_t(1) << 24;  // rows per launch, far below grid limits
  for (int64_t r0 = 0; r0 < rows; r0 += chunk) {
    a.row0 = r0;
    const int64_t blocks = (std::min(chunk, rows - r0) + 3) / 4;
    hipLaunchKernelGGL((append_kernel<P, D, INT8>), dim3(unsigned(blocks)), dim3(256), 0,
                       stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvp

extern "C" kvp_status kvp_kv_append(const kvp_pool* pool, void* k_pool, void* v_pool,
                                    void* k_meta, void* v_meta, const void* k_new,
                                    const void* v_new, const int32_t* seq_idx, const int32_t* pos,
                                    int32_t n_tokens, const int32_t* block_tables,
                                    int32_t num_seqs, int32_t max_blocks, kvp_stream_t stream) {
  using namespace kvp;
  kvp_pool_desc d;
  if (kvp_pool_get_desc(pool, &d) != KVP_OK) return KVP_E_INVAL;
  if (n_tokens < 0 || num_seqs < 0 || max_blocks <= 0) return KVP_E_INVAL;
  if (n_tokens == 0) return KVP_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !seq_idx || !pos || !block_tables)
    return KVP_E_INVAL;
  const bool int8 = d.dtype == KVP_INT8;
  if (int8 != (k_meta != nullptr) || int8 != (v_meta != nullptr)) return KVP_E_INVAL;
  if (int64_t(max_blocks) * d.page_size > 0x7fffffff) return KVP_E_INVAL;
  AppendArgs a{k_pool, v_pool, static_cast<uint16_t*>(k_meta), static_cast<uint16_t*>(v_meta),
               static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
               seq_idx, pos, block_tables, 0, n_tokens, num_seqs, max_blocks, d.num_pages,
               d.num_kv_heads};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  const int key = (d.page_size == 32) * 4 + (d.head_dim == 128) * 2 + int8;
  switch (key) {
    case 0: e = launch_append<16, 64, false>(a, s); break;
    case 1: e = launch_append<16, 64, true>(a, s); break;
    case 2: e = launch_append<16, 128, false>(a, s); break;
    case 3: e = launch_append<16, 128, true>(a, s); break;
    case 4: e = launch_append<32, 64, false>(a, s); break;
    case 5: e = launch_append<32, 64, true>(a, s); break;
    case 6: e = launch_append<32, 128, false>(a, s); break;
    default: e = launch_append<32, 128, true>(a, s); break;
  }
  return e == hipSuccess ? KVP_OK : KVP_E_HIP;
}

// Copy whole pages (every KV head) of one layer's pools: the device half of
// copy-on-write for pages several sequences share ("KV-Cache Optimization
// Techniques", section "Prefix Caching": an existing prefix is reused via
// copy-on-write).  A page occupies page_bytes contiguous bytes of the K pool,
// the same of the V pool, and meta_bytes of each metadata array.  Workgroup
// (pair, part) copies one quarter-page strip of K, V and metadata with 16-byte
// accesses; pairs naming a page outside the pool are skipped.
namespace kvp {

__global__ __launch_bounds__(256) void copy_pages_kernel(char* k, char* v, char* km, char* vm,
                                                         const int32_t* pairs, int32_t n,
                                                         int32_t num_pages, int64_t page_bytes,
                                                         int64_t meta_bytes) {
  const int pair = blockIdx.x >> 2, part = blockIdx.x & 3;
  if (pair >= n) return;
  const int src = pairs[2 * pair], dst = pairs[2 * pair + 1];
  if (unsigned(src) >= unsigned(num_pages) || unsigned(dst) >= unsigned(num_pages) || src == dst)
    return;
  const int64_t strip = page_bytes / 4;  // page bytes are a multiple of 64
  const int64_t s0 = int64_t(src) * page_bytes + part * strip;
  const int64_t d0 = int64_t(dst) * page_bytes + part * strip;
  for (int64_t o = int64_t(threadIdx.x) * 16; o < strip; o += 256 * 16) {
    *reinterpret_cast<uint4*>(k + d0 + o) = *reinterpret_cast<const uint4*>(k + s0 + o);
    *reinterpret_cast<uint4*>(v + d0 + o) = *reinterpret_cast<const uint4*>(v + s0 + o);
  }
  if (km && part == 0) {
    const int64_t ms = int64_t(src) * meta_bytes, md = int64_t(dst) * meta_bytes;
    for (int64_t o = int64_t(threadIdx.x) * 16; o < meta_bytes; o += 256 * 16) {
      *reinterpret_cast<uint4*>(km + md + o) = *reinterpret_cast<const uint4*>(km + ms + o);
      *reinterpret_cast<uint4*>(vm + md + o) = *reinterpret_cast<const uint4*>(vm + ms + o);
    }
  }
}

}  // namespace kvp

extern "C" kvp_status kvp_copy_pages(const kvp_pool* pool, void* k_pool, void* v_pool,
                                     void* k_meta, void* v_meta, const int32_t* src_dst,
                                     int32_t n, kvp_stream_t stream) {
  kvp_pool_desc d;
  if (kvp_pool_get_desc(pool, &d) != KVP_OK || n < 0) return KVP_E_INVAL;
  if (n == 0) return KVP_OK;
  if (!k_pool || !v_pool || !src_dst) return KVP_E_INVAL;
  const bool int8 = d.dtype == KVP_INT8;
  if (int8 != (k_meta != nullptr) || int8 != (v_meta != nullptr)) return KVP_E_INVAL;
  const int64_t elem = int8 ? 1 : 2;
  const int64_t page_bytes = int64_t(d.num_kv_heads) * d.page_size * d.head_dim * elem;
  const int64_t meta_bytes = int8 ? int64_t(d.num_kv_heads) * d.page_size * 4 : 0;
  if (int64_t(n) * 4 > 0x7fffffff) return KVP_E_UNSUPPORTED;
  hipLaunchKernelGGL(kvp::copy_pages_kernel, dim3(unsigned(n) * 4), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<char*>(k_pool),
                     static_cast<char*>(v_pool), static_cast<char*>(k_meta),
                     static_cast<char*>(v_meta), src_dst, n, d.num_pages, page_bytes, meta_bytes);
  return hipGetLastError() == hipSuccess ? KVP_OK : KVP_E_HIP;
}
