"""E4M3 codec of the oracle (test infrastructure only).

The format: 1 sign bit, a 4-bit exponent and a 3-bit mantissa ("FP8
Mixed-Precision Training: Hardware Acceleration Beyond NVIDIA's Paradigm",
section 1.1; "unified E4M3 format" page, section "Fine-Grained Quantization
Strategy").  The variant is OCP E4M3FN: exponent bias 7, subnormals when the
exponent field is 0, no infinities, NaN only for S.1111.111, so the largest
finite magnitude is 1.75 * 2^8 = 448.

decode(b):   S = b>>7, E = (b>>3)&15, F = b&7
             E == 15 and F == 7  -> NaN
             E == 0              -> (-1)^S * F * 2^-9
             otherwise           -> (-1)^S * (8+F) * 2^(E-10)

encode(y):   round |y| to the nearest grid value, ties to the even mantissa,
             saturate at 448 (the pages fix no overflow rule; saturation is
             the reading taken), then put the sign bit of y back, so -0 and
             negative values that round to zero give 0x80.
"""

import numpy as np

E4M3_MAX = 448.0
MIN_NORMAL = 2.0 ** -6


def decode(codes):
    """uint8 codes -> float64 values (NaN for 0x7F and 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = c >> 7
    exp = (c >> 3) & 15
    man = c & 7
    mag = np.where(exp == 0,
                   man.astype(np.float64) * 2.0 ** -9,
                   (8 + man).astype(np.float64) * np.exp2(exp.astype(np.float64) - 10.0))
    val = np.where(sign == 1, -mag, mag)
    return np.where((exp == 15) & (man == 7), np.nan, val)


def encode(y):
    """float32 values -> uint8 E4M3 codes, round-to-nearest-even, saturating.

    Every step is exact in float64: |y| is a float32 value, so |y| * 2^k is
    representable, and ``np.rint`` rounds half to even.
    """
    y = np.asarray(y, dtype=np.float32)
    if np.isnan(y).any():
        raise ValueError("encode: NaN input has no E4M3 code in this reading")
    a = np.abs(y.astype(np.float64))
    sign = np.signbit(y).astype(np.int64) << 7

    # subnormal range, |y| < 2^-6: code = rint(|y| * 2^9); 8 lands on 2^-6 = 0x08
    sub = np.rint(np.minimum(a, 1.0) * 512.0).astype(np.int64)

    # normal range: |y| = m * 2^e with m in [1, 2); r = rint(|y| * 2^(3-e)) in [8, 16]
    safe = np.where(a >= MIN_NORMAL, a, 1.0)
    _, fexp = np.frexp(safe)           # safe = f * 2^fexp, f in [0.5, 1)
    e = fexp.astype(np.int64) - 1
    r = np.rint(np.ldexp(safe, (3 - e).astype(np.int32))).astype(np.int64)
    carry = r == 16
    e = np.where(carry, e + 1, e)
    r = np.where(carry, 8, r)
    norm = ((e + 7) << 3) | (r - 8)

    code = np.where(a < MIN_NORMAL, sub, norm)
    code = np.where(a > E4M3_MAX, 0x7E, code)
    return (code | sign).astype(np.uint8)


def finite_codes():
    """All 254 codes that decode to a number (0x7F and 0xFF excluded)."""
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]
