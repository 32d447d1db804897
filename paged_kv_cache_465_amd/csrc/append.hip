// kv_append: write new K/V rows into the slots their block tables name.
//
// "KV-Cache Optimization Techniques", section "PagedAttention": the page table
// maps a token's logical position to a physical page; position pos sits in
// page block_table[pos / P] at row pos % P.  INT8 pools store each (token, KV
// head) row quantized per token (section "KV-Cache Quantization", eq. 3) with
// a float16 scale and zero point, following the row contract in kvp.h; INT4
// pools the same contract with 4-bit codes, FP8 pools e4m3 codes with a
// per-token scale.
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

// The row contracts, one IEEE float32 operation at a time (no contraction).
// Integer codes (INT8: STEPS = 254, codes -128..127; INT4: STEPS = 14, codes
// -8..7): z = f16((mx+mn)*0.5), s = f16((mx-mn)/STEPS) (1 if 0),
// code = clamp(rint_even((x - z)/s), LO, HI).
template <int E, int STEPS, int LO, int HI>
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
  const float sf = (mx - mn) / float(STEPS);
  _Float16 s16 = (_Float16)sf;
  if (s16 == (_Float16)0.0f) s16 = (_Float16)1.0f;
  const float z = (float)z16, s = (float)s16;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float q = __builtin_rintf((x[e] - z) / s);
    q = fminf(fmaxf(q, float(LO)), float(HI));
    code[e] = (int32_t)q;
  }
  scale_zero = uint32_t(__builtin_bit_cast(uint16_t, s16)) |
               (uint32_t(__builtin_bit_cast(uint16_t, z16)) << 16);
}

// FP8 (e4m3) rows: s = f16(max|x| / 448) (1 if 0), code = e4m3(x / s), zero 0.
template <int E>
__device__ __forceinline__ void quantize_row_fp8(const float (&x)[E], int32_t (&code)[E],
                                                 uint32_t& scale_zero) {
#pragma clang fp contract(off)
  float amax = fabsf(x[0]);
#pragma unroll
  for (int e = 1; e < E; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = wave_max(amax);
  _Float16 s16 = (_Float16)(amax / 448.0f);
  if (s16 == (_Float16)0.0f) s16 = (_Float16)1.0f;
  const float s = (float)s16;
#pragma unroll
  for (int e = 0; e < E; ++e) code[e] = int32_t(f32_to_e4m3(x[e] / s));
  scale_zero = uint32_t(__builtin_bit_cast(uint16_t, s16));
}

template <int P, int D, int F>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int E = D / 64;  // channels per lane
  const int lane = threadIdx.x & 63;
  const int64_t item = a.row0 + int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int H = a.num_kv_heads;
  if (item >= int64_t(a.n_tokens) * H) return;
  const int n = int(item / H), h = int(item % H);
  const int d0 = lane * E;
  const int64_t src = (int64_t(n) * H + h) * D + d0;
  // the new row's values depend only on the row index: load them alongside
  // the position, ahead of the table lookup, so one memory round trip less
  // stands between the launch and the stores
  uint32_t kb[E], vb[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kb[e] = a.k_new[src + e];
    vb[e] = a.v_new[src + e];
  }
  const int sq = a.seq_idx[n], ps = a.pos[n];
  if (sq < 0 || sq >= a.num_seqs || ps < 0 || ps >= a.max_blocks * P) return;
  const int page = a.bt[int64_t(sq) * a.max_blocks + ps / P];
  if (page < 0 || page >= a.num_pages) return;
  const int t = ps % P;
  const int64_t tile = int64_t(page) * H + h;  // (page, head) tile index
  if constexpr (F == kBF16) {
    uint16_t* K = static_cast<uint16_t*>(a.k_pool);
    uint16_t* V = static_cast<uint16_t*>(a.v_pool);
    const int64_t krow = (tile * P + t) * D + d0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      K[krow + e] = uint16_t(kb[e]);
      V[(tile * D + d0 + e) * P + t] = uint16_t(vb[e]);
    }
    return;
  } else {
    float xk[E], xv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      xk[e] = bf16_to_f32(kb[e]);
      xv[e] = bf16_to_f32(vb[e]);
    }
    int32_t ck[E], cv[E];
    uint32_t mk, mv;
    if constexpr (F == kI8) {
      quantize_row<E, 254, -128, 127>(xk, ck, mk);
      quantize_row<E, 254, -128, 127>(xv, cv, mv);
    } else if constexpr (F == kI4) {
      quantize_row<E, 14, -8, 7>(xk, ck, mk);
      quantize_row<E, 14, -8, 7>(xv, cv, mv);
    } else {
      quantize_row_fp8<E>(xk, ck, mk);
      quantize_row_fp8<E>(xv, cv, mv);
    }
    uint8_t* K = static_cast<uint8_t*>(a.k_pool);
    uint8_t* V = static_cast<uint8_t*>(a.v_pool);
    if constexpr (F == kI4) {
      // channel pairs share a byte (even channel in the low nibble, code + 8);
      // K row bytes [t][D/2], V bytes [D/2][t] per (page, head) tile
      constexpr int RB = D / 2;
      if constexpr (E == 2) {
        const uint8_t bk = uint8_t((ck[0] + 8) | ((ck[1] + 8) << 4));
        const uint8_t bv = uint8_t((cv[0] + 8) | ((cv[1] + 8) << 4));
        K[(tile * P + t) * RB + lane] = bk;
        V[(tile * RB + lane) * P + t] = bv;
      } else {
        // one channel per lane: the even lane of each pair writes both nibbles
        const int ok = __shfl_xor(ck[0], 1), ov = __shfl_xor(cv[0], 1);
        if ((lane & 1) == 0) {
          K[(tile * P + t) * RB + (lane >> 1)] = uint8_t((ck[0] + 8) | ((ok + 8) << 4));
          V[(tile * RB + (lane >> 1)) * P + t] = uint8_t((cv[0] + 8) | ((ov + 8) << 4));
        }
      }
    } else {
      const int64_t krow = (tile * P + t) * D + d0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        K[krow + e] = uint8_t(ck[e]);
        V[(tile * D + d0 + e) * P + t] = uint8_t(cv[e]);
      }
    }
    if (lane == 0) {
      const int64_t m = (tile * P + t) * 2;
      *reinterpret_cast<uint32_t*>(a.k_meta + m) = mk;
      *reinterpret_cast<uint32_t*>(a.v_meta + m) = mv;
    }
  }
}

template <int P, int D, int F>
hipError_t launch_append(AppendArgs a, hipStream_t stream) {
  discard_stale_error();
  const int64_t rows = int64_t(a.n_tokens) * a.num_kv_heads;
  const int64_t chunk = int64_t(1) << 24;  // rows per launch, far below grid limits
  for (int64_t r0 = 0; r0 < rows; r0 += chunk) {
    a.row0 = r0;
    const int64_t blocks = (std::min(chunk, rows - r0) + 3) / 4;
    hipLaunchKernelGGL((append_kernel<P, D, F>), dim3(unsigned(blocks)), dim3(256), 0, stream,
                       a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int P, int D>
hipError_t launch_append_fmt(AppendArgs a, int fmt, hipStream_t s) {
  switch (fmt) {
    case kBF16: return launch_append<P, D, kBF16>(a, s);
    case kI8: return launch_append<P, D, kI8>(a, s);
    case kI4: return launch_append<P, D, kI4>(a, s);
    default: return launch_append<P, D, kFP8>(a, s);
  }
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
  const bool quant = d.dtype != KVP_BF16;
  if (quant != (k_meta != nullptr) || quant != (v_meta != nullptr)) return KVP_E_INVAL;
  if (int64_t(max_blocks) * d.page_size > 0x7fffffff) return KVP_E_INVAL;
  AppendArgs a{k_pool, v_pool, static_cast<uint16_t*>(k_meta), static_cast<uint16_t*>(v_meta),
               static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
               seq_idx, pos, block_tables, 0, n_tokens, num_seqs, max_blocks, d.num_pages,
               d.num_kv_heads};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  const int fmt = int(d.dtype);
  if (d.page_size == 16)
    e = d.head_dim == 128 ? launch_append_fmt<16, 128>(a, fmt, s)
                          : launch_append_fmt<16, 64>(a, fmt, s);
  else
    e = d.head_dim == 128 ? launch_append_fmt<32, 128>(a, fmt, s)
                          : launch_append_fmt<32, 64>(a, fmt, s);
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
  const bool quant = d.dtype != KVP_BF16;
  if (quant != (k_meta != nullptr) || quant != (v_meta != nullptr)) return KVP_E_INVAL;
  const int64_t bits = d.dtype == KVP_BF16 ? 16 : (d.dtype == KVP_INT4 ? 4 : 8);
  const int64_t page_bytes = int64_t(d.num_kv_heads) * d.page_size * d.head_dim * bits / 8;
  const int64_t meta_bytes = quant ? int64_t(d.num_kv_heads) * d.page_size * 4 : 0;
  if (int64_t(n) * 4 > 0x7fffffff) return KVP_E_UNSUPPORTED;
  kvp::discard_stale_error();
  hipLaunchKernelGGL(kvp::copy_pages_kernel, dim3(unsigned(n) * 4), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<char*>(k_pool),
                     static_cast<char*>(v_pool), static_cast<char*>(k_meta),
                     static_cast<char*>(v_meta), src_dst, n, d.num_pages, page_bytes, meta_bytes);
  return hipGetLastError() == hipSuccess ? KVP_OK : KVP_E_HIP;
}
