// Device helpers shared by the gfx950 kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvp {

// The runtime keeps the last error of any earlier call on this thread until
// it is read; errors the caller's own calls left behind are not a launch
// failure of this library, so they are read (and dropped) before launching.
inline void discard_stale_error() { (void)hipGetLastError(); }

// True when the predicate holds in any lane of the wavefront (a wave-uniform
// branch condition).
__device__ __forceinline__ bool wave_any(bool pred) {
  return __builtin_amdgcn_ballot_w64(pred) != 0;
}



typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr float kLog2e = 1.4426950408889634f;

// KV storage formats (kvp_kv_dtype values).
enum KvFmt : int { kBF16 = 0, kI8 = 1, kI4 = 2, kFP8 = 3 };

template <int F>
struct FmtInfo {
  static constexpr bool quant = F != kBF16;             // codes + per-token metadata
  static constexpr bool zero = F == kI8 || F == kI4;    // metadata carries a zero point
  static constexpr int bits = F == kBF16 ? 16 : (F == kI4 ? 4 : 8);
  // codes convert to float16 exactly; FP8 codes come out scaled by 2^-8, which
  // this factor (folded into the per-token scale) undoes
  static constexpr float scale_mul = F == kFP8 ? 256.0f : 1.0f;
  // decode's INT4 K operand carries this offset (codes8_to_f16x8_offset)
  static constexpr float koff = F == kI4 ? 1032.0f : 0.0f;
};

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
// of an MFMA 16x16 tile that hold the same column.  The row swaps exchange
// registers between lanes directly (no trip through the LDS crossbar): with
// both operands v, permlane16_swap returns (v of l & ~16, v of l | 16) and
// permlane32_swap (v of l & ~32, v of l | 32) in every lane l.
__device__ __forceinline__ float group4_max(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float group4_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t w = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Power-of-two exponent c for the float16 P.V operands of quantized pools,
// from the largest biased float32 exponent e of the V scales seen so far (0:
// none yet).  V scales are below 2^(e - 126) and softmax weights at most 1,
// so weight * 2^c * scale stays below 2^15 (inside float16, and above its
// subnormals unless the weight itself is tiny) with c = 141 - e; c is capped
// at 100 so that sums of weights times 2^c stay far inside float32's range.
__device__ __forceinline__ int vexp_offset(int e) { return e == 0 ? 0 : min(141 - e, 100); }
// 2^n as a float32 (-126 <= n <= 127)
__device__ __forceinline__ float exp2_int(int n) { return __uint_as_float(uint32_t(n + 127) << 23); }

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

// Four e4m3 codes (one dword) -> float16 values equal to the e4m3 values times
// 2^-8, exactly: moving sign, exponent and mantissa into a float16's fields
// with the exponent bias difference (15 - 7) left out keeps every finite code,
// subnormals included, exact (only the NaN code has no meaning here).
__device__ __forceinline__ void fp8x4_to_f16x4(uint32_t w, f16x2_t& lo, f16x2_t& hi) {
  const uint32_t a = __builtin_amdgcn_perm(0u, w, 0x010c000cu);  // b0 << 8 | b1 << 24
  const uint32_t b = __builtin_amdgcn_perm(0u, w, 0x030c020cu);  // b2 << 8 | b3 << 24
  lo = __builtin_bit_cast(f16x2_t, (a & 0x80008000u) | ((a >> 1) & 0x3f803f80u));
  hi = __builtin_bit_cast(f16x2_t, (b & 0x80008000u) | ((b >> 1) & 0x3f803f80u));
}

// Eight 4-bit codes (one dword; byte j holds channel 2j in its low nibble and
// 2j+1 in its high nibble, each as code + 8) -> eight exact float16 codes in
// the slot order of kI4KSlot: each mask-and-or places two nibbles under the
// float16 exponent of 1024 (low nibbles: 1024 + u; high nibbles: 1024 + 16 u),
// and one packed add or fma per pair removes the offsets.
__device__ __forceinline__ f16x8_t i4x8_to_f16x8(uint32_t w) {
  const uint32_t w8 = w >> 8;
  const f16x2_t a = __builtin_bit_cast(f16x2_t, (w & 0x000f000fu) | 0x64006400u);   // ch 0, 4
  const f16x2_t b = __builtin_bit_cast(f16x2_t, (w & 0x00f000f0u) | 0x64006400u);   // ch 1, 5
  const f16x2_t c = __builtin_bit_cast(f16x2_t, (w8 & 0x000f000fu) | 0x64006400u);  // ch 2, 6
  const f16x2_t d = __builtin_bit_cast(f16x2_t, (w8 & 0x00f000f0u) | 0x64006400u);  // ch 3, 7
  const f16x2_t off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const f16x2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const f16x2_t off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const f16x2_t p0 = a + off, p2 = c + off;
  const f16x2_t p1 = b * sixteenth + off16, p3 = d * sixteenth + off16;
  return f16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}
// Channel (of the dword's eight) in slot e of i4x8_to_f16x8's result.
__device__ __forceinline__ constexpr int kI4KSlot(int e) {
  return (e & 1) * 4 + (e >> 1);
}

// Four bytes, each holding this lane's channel in one nibble (the high one
// when hi_nibble) -> four exact float16 codes, in the token order of
// kV4Slot: lo = tokens (0, 2), hi = tokens (1, 3).  One mask-and-or per pair
// places the nibbles under the float16 exponent of 1024 (a low nibble as
// 1024 + u, a high one as 1024 + 16 u) and one packed fma removes the offset
// (x 1 - 1032, or x 1/16 - 72): exact.
__device__ __forceinline__ void i4sel4_to_f16x4(uint32_t w, bool hi_nibble, f16x2_t& lo,
                                                f16x2_t& hi) {
  const uint32_t mask = hi_nibble ? 0x00f000f0u : 0x000f000fu;
  const f16x2_t mul = hi_nibble ? f16x2_t{(_Float16)0.0625f, (_Float16)0.0625f}
                                : f16x2_t{(_Float16)1.0f, (_Float16)1.0f};
  const f16x2_t off = hi_nibble ? f16x2_t{(_Float16)-72.0f, (_Float16)-72.0f}
                                : f16x2_t{(_Float16)-1032.0f, (_Float16)-1032.0f};
  const f16x2_t a = __builtin_bit_cast(f16x2_t, (w & mask) | 0x64006400u);         // tokens 0, 2
  const f16x2_t b = __builtin_bit_cast(f16x2_t, ((w >> 8) & mask) | 0x64006400u);  // tokens 1, 3
  lo = a * mul + off;
  hi = b * mul + off;
}

// Eight consecutive code channels of a lane (starting at dword w[0]) as the
// float16 matrix-core operand: INT8 and FP8 take two dwords, INT4 one.
template <int F>
__device__ __forceinline__ f16x8_t codes8_to_f16x8(const uint32_t* w) {
  if constexpr (F == kI4) {
    return i4x8_to_f16x8(w[0]);
  } else {
    f16x2_t a0, a1, b0, b1;
    if constexpr (F == kI8) {
      i8x4_to_f16x4(w[0], a0, a1);
      i8x4_to_f16x4(w[1], b0, b1);
    } else {
      fp8x4_to_f16x4(w[0], a0, a1);
      fp8x4_to_f16x4(w[1], b0, b1);
    }
    return f16x8_t{a0[0], a0[1], a1[0], a1[1], b0[0], b0[1], b1[0], b1[1]};
  }
}

// Decode's K operand: for INT4 the eight channels of i4x8_to_f16x8 (same
// slots) as code + 1032, exactly (each nibble u = code + 8 under the float16
// exponent of 1024, `expo`, from three shifts and four mask-and-ors): the
// offset is left in, so the dot product with q carries 1032 sum(q), which
// the caller removes once per dot product instead of once per code.  Other
// formats as codes8_to_f16x8.
template <int F>
__device__ __forceinline__ f16x8_t codes8_to_f16x8_offset(const uint32_t* w,
                                                         uint32_t expo = 0x64006400u) {
  if constexpr (F == kI4) {
    const uint32_t x = w[0];
    const f16x2_t a = __builtin_bit_cast(f16x2_t, (x & 0x000f000fu) | expo);          // ch 0, 4
    const f16x2_t b = __builtin_bit_cast(f16x2_t, ((x >> 4) & 0x000f000fu) | expo);   // ch 1, 5
    const f16x2_t c = __builtin_bit_cast(f16x2_t, ((x >> 8) & 0x000f000fu) | expo);   // ch 2, 6
    const f16x2_t d = __builtin_bit_cast(f16x2_t, ((x >> 12) & 0x000f000fu) | expo);  // ch 3, 7
    return f16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else {
    return codes8_to_f16x8<F>(w);
  }
}

// Four codes of one channel from one dword (a V^T operand): four INT8 or
// FP8 bytes, or for INT4 four bytes of a channel pair with this lane's
// channel in the high nibble when hi_nibble.  Result slot s (lo[0], lo[1],
// hi[0], hi[1]) holds token kV4Slot<F>(s) of the four.
template <int F>
__device__ __forceinline__ constexpr int kV4Slot(int s) {
  return F == kI4 ? ((s & 1) << 1) | (s >> 1) : s;
}
template <int F>
__device__ __forceinline__ void codes4_to_f16x4(uint32_t w, bool hi_nibble, f16x2_t& lo,
                                                f16x2_t& hi) {
  if constexpr (F == kI8)
    i8x4_to_f16x4(w, lo, hi);
  else if constexpr (F == kFP8)
    fp8x4_to_f16x4(w, lo, hi);
  else
    i4sel4_to_f16x4(w, hi_nibble, lo, hi);
}

// float32 -> e4m3 code (OCP e4m3fn: bias 7, 3 mantissa bits, largest finite
// 448, no infinities), round to nearest with ties to the even code,
// magnitudes at or beyond 448 saturating to 448; the sign bit follows y.
// Scaling by powers of two is exact, so each rint sees the exact quotient.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (!(a < 448.0f)) return sign | 0x7eu;
  if (a < 0.015625f) {                             // below 2^-6: steps of 2^-9
    return sign | uint32_t(__builtin_rintf(a * 512.0f));  // 8 is the smallest normal, code 8
  }
  const int e = int((__float_as_uint(a) >> 23) & 0xffu) - 127;  // -6 .. 8
  const float m = __builtin_rintf(a * __uint_as_float(uint32_t(127 + 3 - e) << 23));  // 8 .. 16
  uint32_t code = (uint32_t(e + 7) << 3) + (uint32_t(m) - 8u);  // m == 16 carries into e + 1
  if (code > 0x7eu) code = 0x7eu;
  return sign | code;
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
