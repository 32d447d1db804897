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
