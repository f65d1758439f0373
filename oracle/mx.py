"""MXFP8 numbers for the FP8-expert variant of the layer, in float64.

TEST INFRASTRUCTURE ONLY (same import rule as ``oracle.moe``).

The pages name BF16/FP8 GLM-5.2 artifacts ("Inside GLM" course page,
Release anatomy lesson) but no scaling format.  The format here is
the OCP Microscaling (MX) v1.0 MXFP8 format, written out from its definition:

* element: FP8 E4M3 ("e4m3fn"): sign, 4 exponent bits with bias 7, 3 mantissa
  bits; exponent field 0 holds the subnormals m/8 * 2^-6; the largest finite
  value is 1.75 * 2^8 = 448; the code S.1111.111 is NaN; no infinities;
* block: 32 consecutive elements along the contraction dimension share one
  scale;
* scale: E8M0, the power of two 2^(code - 127) (code 255 is NaN, unused).

Quantisation of a block (a reading: the MX specification leaves the choice
of the shared exponent to the implementation): the scale is the smallest
power of two 2^s with max|v| <= 448 * 2^s, so no element saturates; each
element is v / 2^s rounded to the nearest E4M3 value, ties to the even
mantissa.  An all-zero block gets scale 2^0 and zero codes.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 32


def decode_e4m3(codes) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values (NaN for the NaN codes)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def encode_e4m3(v) -> np.ndarray:
    """Nearest E4M3 code (ties to even mantissa) of finite |v| <= 448."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.abs(v) <= E4M3_MAX):
        raise ValueError("value outside the E4M3 range")
    a = np.abs(v)
    # exponent of the binade holding a (subnormal binade below 2^-6)
    _, x = np.frexp(a)                      # a = f * 2^x, f in [0.5, 1)
    eu = np.maximum(x - 1, -6)              # unbiased exponent, at least -6
    step = np.ldexp(1.0, eu - 3)            # spacing of E4M3 values in that binade
    q = np.round(a / step)                  # numpy rounds halves to even
    # normal binade: q in [8, 16]; q == 16 moves to the next binade (code +8
    # works out the same because codes are contiguous); subnormal: q in [0, 8]
    field = np.where(eu == -6, 0, eu + 7)   # exponent field of the binade start
    code = np.where(eu == -6, q, (field << 3) + (q - 8)).astype(np.int64)
    code = np.where(a == 0, 0, code)
    return (code | np.where(np.signbit(v) & (a != 0), 0x80, 0)).astype(np.uint8)


def block_exponent(amax) -> np.ndarray:
    """Smallest integer s with amax <= 448 * 2^s (0 where amax == 0).

    Exact: with amax = f * 2^x (f in [0.5, 1)) and 448 = 0.875 * 2^9, the
    condition reads f / 0.875 <= 2^(9 + s - x); s = x - 9 when f <= 0.875,
    else x - 8.
    """
    amax = np.asarray(amax, dtype=np.float64)
    f, x = np.frexp(amax)
    s = np.where(f <= 0.875, x - 9, x - 8)
    return np.where(amax == 0, 0, s).astype(np.int64)


def quantize(v, block: int = BLOCK):
    """MXFP8 encoding along the last axis -> (E4M3 codes uint8, E8M0 scales uint8).

    The last axis length must be a multiple of ``block``.
    """
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    if n % block:
        raise ValueError("last axis is not a multiple of the block size")
    vb = v.reshape(v.shape[:-1] + (n // block, block))
    s = block_exponent(np.abs(vb).max(axis=-1))
    if np.any(s + 127 < 0) or np.any(s + 127 > 254):
        raise ValueError("block scale outside the E8M0 range")
    codes = encode_e4m3(vb / np.ldexp(1.0, s)[..., None])
    return codes.reshape(v.shape), (s + 127).astype(np.uint8)


_E4M3_VALUES = decode_e4m3(np.arange(256))   # every code's value, from the definition above


def dequantize(codes, scales, block: int = BLOCK) -> np.ndarray:
    """Values of MXFP8 data: decode(code) * 2^(scale - 127) per block."""
    c = _E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]
    n = c.shape[-1]
    s = np.asarray(scales).astype(np.int64) - 127
    cb = c.reshape(c.shape[:-1] + (n // block, block))
    return (cb * np.ldexp(1.0, s)[..., None]).reshape(c.shape)


def fake_quantize(v, block: int = BLOCK) -> np.ndarray:
    """The values an MXFP8 encoding of ``v`` represents."""
    return dequantize(*quantize(v, block), block)
