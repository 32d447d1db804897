// Streaming-read probe: the HBM read rate of the decode kernels' access
// pattern with no arithmetic behind it.
//
// Paged decode attention reads each (page, KV head) tile of K and of V once
// per step ("KV Cache Optimization" glossary, section "Memory-Bound
// Operation": decode is limited by memory bandwidth, not compute).  Each tile
// is a contiguous chunk (4 KiB for 16 tokens x 128 channels of bfloat16) at a
// position the block table shuffles.  This kernel reads chunks of two
// buffers (a K-like and a V-like pool) in the order a device array of chunk
// ids gives, with the decode kernels' loads (16 bytes per lane, non-temporal
// hint) and a ring of chunks in flight per wavefront, and folds what
// it read into one word per lane so no load can be dropped.  With the decode
// kernels' depth and wavefront count its rate is the ceiling their page
// streaming can reach; other depths and counts show what the part allows.
#include "device_common.h"
#include "kvp.h"

namespace kvp {

// One wavefront per stream of chunks: chunks [w*per, (w+1)*per) of the id
// list, each read from both buffers; LOADS 16-byte loads per lane per chunk
// per buffer (chunk_bytes = LOADS * 1024), DEPTH chunks in flight.
template <int LOADS, int DEPTH>
__global__ __launch_bounds__(256) void probe_read_kernel(const char* __restrict__ a,
                                                         const char* __restrict__ b,
                                                         int64_t n_pool_chunks,
                                                         const int32_t* __restrict__ ids,
                                                         int32_t n_chunks, int32_t per_wave,
                                                         int32_t n_waves,
                                                         uint32_t* __restrict__ sink) {
  constexpr int CHUNK = LOADS * 1024;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (w >= n_waves) return;
  const int c0 = w * per_wave;
  const int c1 = min(c0 + per_wave, n_chunks);
  uint32_t acc = 0;
  auto fold = [&](const uint4& v) { acc ^= v.x ^ v.y ^ v.z ^ v.w; };
  uint4 ra[DEPTH][LOADS], rb[DEPTH][LOADS];
  auto issue = [&](int slot, int c) {
    int id = ids[min(c, c1 - 1)];
    id = (id >= 0 && id < n_pool_chunks) ? id : 0;   // ids outside the buffers read chunk 0
    const char* pa = a + int64_t(id) * CHUNK + lane * 16;
    const char* pb = b + int64_t(id) * CHUNK + lane * 16;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      ra[slot][i] = load_stream<uint4>(pa + i * 1024);
      rb[slot][i] = load_stream<uint4>(pb + i * 1024);
    }
  };
  if (c1 > c0) {
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) issue(s, c0 + s);
    for (int c = c0; c < c1; c += DEPTH) {
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) {
        if (c + s < c1) {
#pragma unroll
          for (int i = 0; i < LOADS; ++i) {
            fold(ra[s][i]);
            fold(rb[s][i]);
          }
        }
        issue(s, c + s + DEPTH);   // past the end: the last chunk again (a cache hit)
      }
    }
#pragma unroll
    for (int s = 0; s < DEPTH; ++s)
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        fold(ra[s][i]);
        fold(rb[s][i]);
      }
  }
  sink[int64_t(w) * 64 + lane] = acc;
}

template <int LOADS>
hipError_t launch_probe(int depth, dim3 grid, hipStream_t s, const char* a, const char* b,
                        int64_t pool_chunks, const int32_t* ids, int32_t n, int32_t per,
                        int32_t waves, uint32_t* sink) {
  switch (depth) {
    case 1:
      hipLaunchKernelGGL((probe_read_kernel<LOADS, 1>), grid, dim3(256), 0, s, a, b, pool_chunks,
                         ids, n, per, waves, sink);
      break;
    case 2:
      hipLaunchKernelGGL((probe_read_kernel<LOADS, 2>), grid, dim3(256), 0, s, a, b, pool_chunks,
                         ids, n, per, waves, sink);
      break;
    case 4:
      hipLaunchKernelGGL((probe_read_kernel<LOADS, 4>), grid, dim3(256), 0, s, a, b, pool_chunks,
                         ids, n, per, waves, sink);
      break;
    default:
      hipLaunchKernelGGL((probe_read_kernel<LOADS, 8>), grid, dim3(256), 0, s, a, b, pool_chunks,
                         ids, n, per, waves, sink);
      break;
  }
  return hipGetLastError();
}

}  // namespace kvp

extern "C" kvp_status kvp_probe_read_chunks(const void* pool_a, const void* pool_b,
                                            size_t pool_bytes, const int32_t* chunk_ids,
                                            int32_t n_chunks, int32_t chunk_bytes,
                                            int32_t chunks_in_flight, int32_t num_waves,
                                            uint32_t* sink, kvp_stream_t stream) {
  using namespace kvp;
  if (n_chunks < 0 || num_waves <= 0) return KVP_E_INVAL;
  if (chunk_bytes != 1024 && chunk_bytes != 2048 && chunk_bytes != 4096 && chunk_bytes != 8192)
    return KVP_E_UNSUPPORTED;
  const int d = chunks_in_flight;
  if (d != 1 && d != 2 && d != 4 && d != 8) return KVP_E_UNSUPPORTED;
  if (chunk_bytes == 8192 && d == 8) return KVP_E_UNSUPPORTED;   // registers
  if (n_chunks == 0) return KVP_OK;
  if (!pool_a || !pool_b || !chunk_ids || !sink || pool_bytes < size_t(chunk_bytes))
    return KVP_E_INVAL;
  const int64_t pool_chunks = int64_t(pool_bytes / size_t(chunk_bytes));
  const int32_t per = (n_chunks + num_waves - 1) / num_waves;
  const dim3 grid(static_cast<unsigned>((num_waves + 3) / 4));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  discard_stale_error();
  const char* a = static_cast<const char*>(pool_a);
  const char* b = static_cast<const char*>(pool_b);
  hipError_t e;
  switch (chunk_bytes) {
    case 1024: e = launch_probe<1>(d, grid, s, a, b, pool_chunks, chunk_ids, n_chunks, per,
                                   num_waves, sink); break;
    case 2048: e = launch_probe<2>(d, grid, s, a, b, pool_chunks, chunk_ids, n_chunks, per,
                                   num_waves, sink); break;
    case 4096: e = launch_probe<4>(d, grid, s, a, b, pool_chunks, chunk_ids, n_chunks, per,
                                   num_waves, sink); break;
    default: e = launch_probe<8>(d, grid, s, a, b, pool_chunks, chunk_ids, n_chunks, per,
                                 num_waves, sink); break;
  }
  return e == hipSuccess ? KVP_OK : KVP_E_HIP;
}
