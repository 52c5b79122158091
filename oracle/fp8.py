"""8-bit floating point (OCP E4M3) KV-cache codes.  TEST INFRASTRUCTURE ONLY.

The pages say only that the KV cache can be kept quantised, FP8 among the
formats ("理解 vLLM PagedAttention", version matrix, row "量化").  The readings
this oracle fixes:

* Format: OCP 8-bit floating point E4M3 ("E4M3FN"): 1 sign bit, 4 exponent bits
  with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals
  m * 2^-9; exponent field 15 with mantissa 7 is NaN; no infinities; the
  largest finite magnitude is 1.75 * 2^8 = 448.
* Scales: one float32 scale per KV head for K and one for V (as the caller
  gives them).  A stored code is  encode(fp32(x) / fp32(scale))  -- the
  division rounded to float32, as the kernel computes it -- and the value it
  stands for is  decode(code) * scale.
* Encoding rounds to nearest, ties to even; magnitudes above 448 (infinities
  included) saturate to 448; NaN encodes as 0x7F.
"""

from __future__ import annotations

import numpy as np

BIAS = 7
MAX_FINITE = 448.0
NAN_CODE = 0x7F


def decode(codes) -> np.ndarray:
    """float64 values of uint8 E4M3 codes (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * np.ldexp(1.0 + m / 8.0, e - BIAS)
    subnormal = sign * np.ldexp(m.astype(np.float64), 1 - BIAS - 3)   # m * 2^-9
    out = np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (m == 7), np.nan, out)


def encode(x) -> np.ndarray:
    """uint8 E4M3 codes of float values: round to nearest even, saturate at 448."""
    v = np.asarray(x, dtype=np.float64)
    nan = np.isnan(v)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    a = np.minimum(np.abs(np.where(nan, 0.0, v)), MAX_FINITE)
    _, exp = np.frexp(a)                       # a = f * 2^exp with f in [0.5, 1)
    e = exp.astype(np.int64) - 1               # a = (2 f) * 2^e, 2 f in [1, 2)
    # below 2^-6: subnormal, quantum 2^-9; m = 8 there is the first normal (code 0x08)
    m_sub = np.rint(a / 2.0 ** (1 - BIAS - 3)).astype(np.int64)
    # normal: 3-bit mantissa of a / 2^e, rounded half to even, with the carry into e
    m = np.rint((np.ldexp(a, -e) - 1.0) * 8.0).astype(np.int64)
    e = np.where(m == 8, e + 1, e)
    m = np.where(m == 8, 0, m)
    normal = ((e + BIAS) << 3) | m
    code = np.where(a < 2.0 ** (1 - BIAS), m_sub, normal) | sign
    return np.where(nan, NAN_CODE, code).astype(np.uint8)


def quantize(x, scale) -> np.ndarray:
    """Codes of x [..., D] with one float32 scale per leading-head index broadcast by the
    caller: encode(fp32(x) / fp32(scale)) with the division in float32."""
    q = np.asarray(x, dtype=np.float32) / np.asarray(scale, dtype=np.float32)
    return encode(q.astype(np.float32))


def dequantize(codes, scale) -> np.ndarray:
    """float64 values decode(code) * scale."""
    return decode(codes) * np.asarray(scale, dtype=np.float32).astype(np.float64)
