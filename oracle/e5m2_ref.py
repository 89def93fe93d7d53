"""E5M2 (OCP) codec, written from its definition.  TEST INFRASTRUCTURE ONLY.

The FP8 cache of [PA/related] ("PagedAttention", section "Các kỹ thuật liên
quan") stores keys and values in 8 bits without naming a format.  Besides E4M3
(``e4m3_ref``) the library offers the OCP specification's other 8-bit format,
E5M2, with one fp32 scale per pool or per kv head:

* bit layout  s eeeee mm, exponent bias 15;
* e == 0            -> subnormal  (-1)^s * 2^-14 * (m / 4)
* 0 < e < 31        -> normal     (-1)^s * 2^(e-15) * (1 + m / 4)   (max 57344)
* e == 31, m == 0   -> infinity;  e == 31, m != 0 -> NaN

Encoding reading (proposed, mirroring the E4M3 one):
  code = nearest_e5m2( saturate( fp32(x) / fp32(scale) ) )
with the IEEE single-precision division, saturation to [-57344, 57344] (so the
cache never stores an infinity), ties to the even mantissa, and NaN -> 0x7F with
the input's sign bit.  Decoding: value = decode(code) * fp32(scale), in float64.
"""

import numpy as np

E5M2_MAX = 57344.0


def _decode_one(code):
    s = (code >> 7) & 1
    e = (code >> 2) & 0x1F
    m = code & 0x3
    sign = -1.0 if s else 1.0
    if e == 0x1F:
        return sign * float("inf") if m == 0 else float("nan")
    if e == 0:
        return sign * (2.0 ** -14) * (m / 4.0)
    return sign * (2.0 ** (e - 15)) * (1.0 + m / 4.0)


_DECODE_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)
_POS_CODES = np.arange(0x00, 0x7C, dtype=np.int64)          # finite non-negative codes, increasing
_POS_VALUES = _DECODE_TABLE[:0x7C]


def decode_e5m2(codes):
    """Decode uint8 codes to float64 values."""
    return _DECODE_TABLE[np.asarray(codes, dtype=np.uint8).astype(np.int64)]


def _nearest_code_nonneg(a):
    """For float64 magnitudes 0 <= a <= 57344: nearest E5M2 code, ties to even mantissa."""
    a = np.asarray(a, dtype=np.float64)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick_hi = np.where(d_hi == d_lo, (_POS_CODES[hi] & 1) == 0, d_hi < d_lo)
    exact = _POS_VALUES[hi] == a
    return np.where(pick_hi | exact, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)


def encode_e5m2(x, scale):
    """Encode values to E5M2 codes: nearest(saturate(fp32(x) / fp32(scale)))."""
    xf = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        q = (xf / np.float32(scale)).astype(np.float32)
    neg = np.signbit(xf)
    isnan = np.isnan(xf)
    mag = np.where(isnan, 0.0, np.minimum(np.abs(q.astype(np.float64)), E5M2_MAX))
    code = _nearest_code_nonneg(mag)
    code = np.where(neg, code | 0x80, code).astype(np.uint8)
    return np.where(isnan, np.where(neg, 0xFF, 0x7F), code).astype(np.uint8)


def dequant_e5m2(codes, scale):
    """Stored value of an E5M2 cache entry: decoded code times the fp32 scale (float64)."""
    return decode_e5m2(codes) * np.float64(np.float32(scale))


def dequant_per_head(codes, scales, decode):
    """A pool ``[NB, KVH, bs, d]`` of codes with one fp32 scale per kv head (float64)."""
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    return decode(codes) * s[None, :, None, None]
