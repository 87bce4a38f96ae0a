"""OCP FP8 E4M3 ("e4m3fn") codec, written from the format's definition.

Test infrastructure (see the package docstring): nothing in the product
path imports this module.

The temporal cache is stored in FP8 while weights and activations stay in
bf16 (PersonaPlex 7B page, section "Compressing the Temporal KV cache").  The
pages name FP8 but no variant; the format used here is OCP E4M3, the
variant with a single NaN pattern and no infinities:

* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
* exponent field 0 encodes subnormals m * 2^-9 (m = 0..7);
* exponent field 15 with mantissa 7 is NaN (both signs); every other code
  is finite, so the largest magnitude is 1.75 * 2^8 = 448;
* encoding rounds to nearest with ties to the even mantissa and saturates
  finite values beyond 448 to +-448 ("satfinite"); NaN maps to 0x7F with the
  input's sign bit.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _decode_code(c: int) -> float:
    sign = -1.0 if (c >> 7) & 1 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# 256-entry decode table built from the format definition (float64; every
# entry is exactly representable in float32).
DECODE_TABLE = np.array([_decode_code(c) for c in range(256)], dtype=np.float64)
DECODE_TABLE_F32 = DECODE_TABLE.astype(np.float32)


def decode(codes: np.ndarray, dtype=np.float32) -> np.ndarray:
    """Exact decode of uint8 codes through the table."""
    t = DECODE_TABLE_F32 if dtype == np.float32 else DECODE_TABLE.astype(dtype)
    return t[np.asarray(codes, dtype=np.uint8)]


def encode(x: np.ndarray) -> np.ndarray:
    """Round float32 values to E4M3 codes (nearest, ties to even, satfinite).

    The arithmetic is exact: the input is widened to float64, the exponent
    is taken with frexp and the scaled significand is rounded with rint,
    which rounds halves to even.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    code = np.zeros(a.shape, dtype=np.int64)

    sat = a >= E4M3_MAX
    sub = a < 2.0 ** -6
    norm = ~(sat | sub)

    # Subnormal range: multiples of 2^-9; rint(a * 2^9) lands in 0..8 and
    # the value 8 is exactly the smallest normal's code 0x08.
    code = np.where(sub, np.rint(np.where(sub, a, 0.0) * 2.0 ** 9).astype(np.int64), code)

    # Normal range: a = f * 2^ex with f in [0.5, 1), so the unbiased
    # exponent is ex - 1 and the significand is 2f in [1, 2).
    f, ex = np.frexp(np.where(norm, a, 1.0))
    e = ex.astype(np.int64) - 1
    m = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    ncode = ((e + 7) << 3) | m
    code = np.where(norm, ncode, code)
    # Rounding can carry 1.75*2^8 < a < 448 only up to 448 itself (the
    # values that would round past it are >= 448 and saturate above).
    code = np.where(sat, 0x7E, code)
    code = np.where(nan, 0x7F, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quantize(x: np.ndarray, scale) -> np.ndarray:
    """Codes of x / scale (float32 division, then encode)."""
    x = np.asarray(x, dtype=np.float32)
    return encode(x / np.float32(scale) if np.isscalar(scale) else x / scale.astype(np.float32))


def dequantize(codes: np.ndarray, scale, dtype=np.float32) -> np.ndarray:
    """scale * decode(codes), in ``dtype``."""
    return decode(codes, dtype) * np.asarray(scale, dtype=dtype)
