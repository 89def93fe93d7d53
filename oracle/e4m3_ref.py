"""E4M3 (OCP "FN" variant) codec, written from its definition.  TEST INFRASTRUCTURE ONLY.

The FP8 cache of [PA/related] ("PagedAttention", section "Các kỹ thuật liên
quan") stores keys and values in 8 bits; the pages say nothing more.  The
workload fixes E4M3 with one fp32 scale per tensor.  The format itself is the
OCP 8-bit floating point specification's E4M3:

* bit layout  s eeee mmm, exponent bias 7;
* e == 0            -> subnormal  (-1)^s * 2^-6 * (m / 8)
* 0 < e < 15        -> normal     (-1)^s * 2^(e-7) * (1 + m / 8)
* e == 15, m < 7    -> normal as above (values 256 .. 448)
* e == 15, m == 7   -> NaN   (there is no infinity)

Encoding reading (proposed; the pages are silent):
  code = nearest_e4m3( saturate( fp32(x) / fp32(scale) ) )
where the division is the IEEE-754 single-precision division, ``saturate``
clamps to [-448, 448] (so +-inf -> +-448), ``nearest_e4m3`` picks the finite
E4M3 value nearest to the quotient with ties going to the code whose mantissa
is even, and NaN maps to the NaN code 0x7F with the input's sign bit (0x7F or
0xFF).  Negative zero keeps its sign (0x80).
Decoding reading:  value = fp32(decode(code)) * fp32(scale)  (evaluated here in
float64, which holds the product exactly).
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN_POS = 0x7F


def _decode_one(code):
    """Value of one E4M3 code per the bit-layout definition (float, NaN for S.1111.111)."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    sign = -1.0 if s else 1.0
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (2.0 ** -6) * (m / 8.0)
    return sign * (2.0 ** (e - 7)) * (1.0 + m / 8.0)


# Table of all 256 decoded values, built once from the definition above.
_DECODE_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)

# Non-negative finite codes in increasing value (codes 0x00 .. 0x7E are monotone).
_POS_CODES = np.arange(0x00, 0x7F, dtype=np.int64)
_POS_VALUES = _DECODE_TABLE[:0x7F]


def decode_e4m3(codes):
    """Decode uint8 codes to float64 values (NaN for the two NaN codes)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _DECODE_TABLE[codes.astype(np.int64)]


def _nearest_code_nonneg(a):
    """For float64 magnitudes 0 <= a <= 448: nearest E4M3 code, ties to even mantissa.

    Plain definition: compare the distance to the next value below and the next
    value above; the smaller distance wins, and on an exact tie the code with an
    even mantissa (lowest bit 0) wins.
    """
    a = np.asarray(a, dtype=np.float64)
    hi = np.searchsorted(_POS_VALUES, a, side="left")       # first value >= a
    hi = np.clip(hi, 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    v_hi = _POS_VALUES[hi]
    v_lo = _POS_VALUES[lo]
    d_hi = v_hi - a
    d_lo = a - v_lo
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    even_hi = (_POS_CODES[hi] & 1) == 0
    pick_hi = np.where(tie, even_hi, pick_hi)
    exact = v_hi == a
    code = np.where(pick_hi | exact, _POS_CODES[hi], _POS_CODES[lo])
    return code.astype(np.uint8)


def encode_e4m3(x, scale):
    """Encode values to E4M3 codes: nearest(saturate(fp32(x) / fp32(scale))).

    ``x`` may be any float array (fp16/bf16 values given as float32/float64 hold
    them exactly); it is first rounded to float32, then divided by the float32
    scale in float32 (IEEE single division, as numpy does it).
    """
    xf = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        q = (xf / np.float32(scale)).astype(np.float32)
    neg = np.signbit(xf)             # scale > 0: the quotient has the input's sign
    isnan = np.isnan(xf)
    mag = np.abs(q.astype(np.float64))
    mag = np.where(isnan, 0.0, np.minimum(mag, E4M3_MAX))
    code = _nearest_code_nonneg(mag)
    code = np.where(neg, code | 0x80, code).astype(np.uint8)
    nan_code = np.where(neg, 0xFF, E4M3_NAN_POS).astype(np.uint8)
    return np.where(isnan, nan_code, code).astype(np.uint8)


def dequant_e4m3(codes, scale):
    """Stored value of an E4M3 cache entry: decoded code times the fp32 scale (float64)."""
    return decode_e4m3(codes) * np.float64(np.float32(scale))
