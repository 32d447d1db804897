"""INT8 per-token KV quantization -- CPU oracle (test infrastructure only).

"KV-Cache Optimization Techniques", section "KV-Cache Quantization", eq. 3:
codes are round((K - z) / s) and the value is recovered as s * code + z; the
per-token calibration gives one scale and one zero point per row.  The page
fixes neither how s and z are chosen nor the rounding mode; the reading taken
here (also the library's documented contract):

* one row = the D channels of one token for one KV head;
* z = midpoint of the row's range, s = range / 254, both stored as float16
  (round to nearest even); s = 1 when it rounds to 0;
* codes = clamp(round_half_even((x - z) / s), -128, 127) computed with the
  float16-rounded s and z, every step an IEEE float32 operation.

numpy's float32 arithmetic rounds each operation to nearest even, np.rint
rounds half to even and astype(float16) rounds to nearest even, so this is
the float32 computation written out.  Pinned by the round-trip bound
|x - (s*code + z)| <= s/2 (plus float32 slack), tie rows and exact-grid rows.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact: bfloat16 is float32's top half)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_rows(x_bits: np.ndarray):
    """Quantize rows of bfloat16 bits, last axis = one row of D channels.

    Returns (codes int8 [..., D], scale_f16_bits uint16 [...], zero_f16_bits uint16 [...]).
    """
    x = bf16_bits_to_f32(x_bits)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    z16 = ((mx + mn) * np.float32(0.5)).astype(np.float16)
    s16 = ((mx - mn) / np.float32(254.0)).astype(np.float16)
    s16 = np.where(s16 == np.float16(0.0), np.float16(1.0), s16)
    zf = z16.astype(np.float32)[..., None]
    sf = s16.astype(np.float32)[..., None]
    q = np.rint((x - zf) / sf)
    codes = np.clip(q, -128, 127).astype(np.int8)
    return codes, s16.view(np.uint16), z16.view(np.uint16)


def dequantize(codes: np.ndarray, scale_bits: np.ndarray, zero_bits: np.ndarray) -> np.ndarray:
    """Stored INT8 row -> float64 values s*code + z (exact in float64)."""
    s = np.asarray(scale_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    z = np.asarray(zero_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    return s[..., None] * codes.astype(np.float64) + z[..., None]


# ---- 4-bit codes (eq. 3 with INT4, section "KV-Cache Quantization": FP16 -> INT4 is 4x) ----
def quantize_rows_int4(x_bits: np.ndarray):
    """The row contract with 4-bit codes: z = f16((mx + mn) * 0.5),
    s = f16((mx - mn) / 14) (1 if it rounds to 0), codes =
    clamp(rint_even((x - z) / s), -8, 7), every step float32 RNE.  Returns
    (codes int8 in -8..7 [..., D], scale bits, zero bits)."""
    x = bf16_bits_to_f32(x_bits)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    z16 = ((mx + mn) * np.float32(0.5)).astype(np.float16)
    s16 = ((mx - mn) / np.float32(14.0)).astype(np.float16)
    s16 = np.where(s16 == np.float16(0.0), np.float16(1.0), s16)
    q = np.rint((x - z16.astype(np.float32)[..., None]) / s16.astype(np.float32)[..., None])
    return np.clip(q, -8, 7).astype(np.int8), s16.view(np.uint16), z16.view(np.uint16)


# ---- FP8 e4m3 (OCP "e4m3fn": 4 exponent bits, bias 7, 3 mantissa bits, largest
# finite 448, no infinities, NaN = S.1111.111) with a per-token scale ----------------
def e4m3_table() -> np.ndarray:
    """float64 value of every code 0..255 (NaN for the two NaN codes)."""
    vals = np.empty(256)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 0xF, code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * m * 2.0 ** -9          # subnormal: m * 2^(1-7) / 8
        else:
            vals[code] = sign * (1 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = e4m3_table()
_E4M3_POS = _E4M3[:0x7F]          # codes 0x00..0x7E: 0 .. 448, increasing


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3fn code to each float (exact comparison in float64), ties
    to the even code (even last mantissa bit), magnitudes beyond 448
    saturating to 448; the sign bit follows x (so -0.0 -> 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


def quantize_rows_fp8(x_bits: np.ndarray):
    """Per-token FP8: s = f16(amax / 448) (1 if it rounds to 0) with float32
    division, codes = e4m3(x / s) with x / s in float32.  Returns (codes uint8
    [..., D], scale bits, zero bits = 0)."""
    x = bf16_bits_to_f32(x_bits)
    amax = np.abs(x).max(axis=-1)
    with np.errstate(over="ignore"):   # beyond float16's range the scale is inf (codes +-0)
        s16 = (amax / np.float32(448.0)).astype(np.float16)
    s16 = np.where(s16 == np.float16(0.0), np.float16(1.0), s16)
    y = x / s16.astype(np.float32)[..., None]
    return e4m3_encode(y), s16.view(np.uint16), np.zeros(s16.shape, dtype=np.uint16)


def dequantize_fp8(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Stored FP8 row -> float64 values s * e4m3(code) (exact)."""
    s = np.asarray(scale_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    return s[..., None] * _E4M3[np.asarray(codes, dtype=np.uint8)]
