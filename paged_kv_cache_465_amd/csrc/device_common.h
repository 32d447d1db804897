// Device helpers shared by the gfx950 kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvp {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr float kLog2e = 1.4426950408889634f;

// Streaming loads of K/V page data: every byte is read once per decode step,
// so the loads carry the non-temporal hint and do not displace reusable lines
// (q, block tables) in L2 and the Infinity Cache.
template <typename T> __device__ __forceinline__ T load_stream(const void* p);
template <> __device__ __forceinline__ uint4 load_stream<uint4>(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <> __device__ __forceinline__ uint2 load_stream<uint2>(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load(static_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
template <> __device__ __forceinline__ uint32_t load_stream<uint32_t>(const void* p) {
  return __builtin_nontemporal_load(static_cast<const uint32_t*>(p));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bfloat16 bits, round to nearest even (quiet NaN preserved).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}

// Reduce over the four 16-lane groups (lanes l, l^16, l^32, l^48): the lanes
// of an MFMA 16x16 tile that hold the same column.
__device__ __forceinline__ float group4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}

__device__ __forceinline__ float group4_sum(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Four signed int8 codes (one dword) -> four exact float16 values.
// fp16 bits 0x6400|u are 1024 + u for u < 1024; with u = code + 128 (the
// sign bit flipped) subtracting 1152 gives the code exactly.
__device__ __forceinline__ void i8x4_to_f16x4(uint32_t w, f16x2_t& lo, f16x2_t& hi) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const f16x2_t off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  lo = __builtin_bit_cast(f16x2_t, a) + off;
  hi = __builtin_bit_cast(f16x2_t, b) + off;
}

__device__ __forceinline__ f32x4_t mfma_16x16x32(const bf16x8_t& a, const bf16x8_t& b,
                                                 const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_16x16x32(const f16x8_t& a, const f16x8_t& b,
                                                 const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_16x16x16(const bf16x4_t& a, const bf16x4_t& b,
                                                 const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_16x16x16(const f16x4_t& a, const f16x4_t& b,
                                                 const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

}  // namespace kvp
