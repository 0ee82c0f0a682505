"""Number formats used by the segment-attention cache (oracle, test-only).

bf16: 1 sign, 8 exponent, 7 stored mantissa bits (the fp32 exponent range).
The pages state that the single-GPU preset stores the KV cache in a narrow
format and computes in BF16 ("El preset de una GPU", inferencekey.com;
"The 4090 preset", ai.thesatyajit.com). Rounding is round-to-nearest, ties to
even, which is the IEEE default.

e4m3fn (OCP 8-bit float, "FN" = finite, no infinities): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits. Exponent field 0 is subnormal
(m * 2**-9); exponent field 15 with mantissa 7 is NaN; everything else is
normal, (1 + m/8) * 2**(e - 7). Largest finite magnitude 448. Encoding rounds
to nearest, ties to even, and saturates magnitudes beyond 448 to 448.
"""

import numpy as np

BF16_MANT_BITS = 7          # stored mantissa bits of bf16
BF16_MIN_NORMAL_EXP = -126  # same exponent range as fp32

E4M3_BIAS = 7
E4M3_MAX = 448.0


def bf16_round(x):
    """Round real values (float64 array) to the nearest bf16 value, ties to even.

    Returns float64 values that are exactly representable in bf16. Works
    directly from the float64 value (no intermediate float32 rounding), so it
    is the correctly rounded bf16 of the exact input. Magnitudes beyond the
    largest bf16 become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    _, e = np.frexp(xf)                 # xf = m * 2**e, 0.5 <= |m| < 1
    lead = np.maximum(e - 1, BF16_MIN_NORMAL_EXP)
    ulp = np.ldexp(1.0, lead - BF16_MANT_BITS)
    r = np.rint(xf / ulp) * ulp         # np.rint rounds half to even
    max_bf16 = (2.0 - 2.0 ** -BF16_MANT_BITS) * 2.0 ** 127
    r = np.where(np.abs(r) > max_bf16, np.sign(r) * np.inf, r)
    out[finite] = r
    out[~finite] = x[~finite]
    return out


def bf16_bits(x):
    """uint16 bit patterns of values that are already exactly bf16."""
    f32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(bits):
    """float64 values of uint16 bf16 bit patterns."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def e4m3_decode(codes):
    """float64 value of each e4m3fn code (uint8), NaN for the NaN codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m * 2.0 ** (1 - E4M3_BIAS - 3)                   # m/8 * 2**(1-7)
    nor = (1.0 + m / 8.0) * np.ldexp(1.0, e - E4M3_BIAS)
    val = np.where(e == 0, sub, nor)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_encode(x):
    """Round float64 values to e4m3fn codes: nearest, ties to even, saturating.

    The inputs are treated as exact reals (callers pass float32-valued
    float64 when they model a float32 decision). NaN maps to 0x7F.
    """
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, np.abs(x))
    codes = np.zeros(x.shape, dtype=np.int64)
    # subnormal range (below 2**-6): grid step 2**-9; code 8 == 2**-6 exactly.
    small = a < 2.0 ** -6
    codes = np.where(small, np.rint(a / 2.0 ** -9), codes)
    big = ~small
    ab = np.where(big, a, 1.0)
    _, e = np.frexp(ab)
    lead = e - 1                                       # 2**lead <= a < 2**(lead+1)
    mant = np.rint((ab / np.ldexp(1.0, lead) - 1.0) * 8.0)
    carry = mant >= 8
    lead = np.where(carry, lead + 1, lead)
    mant = np.where(carry, 0, mant)
    ncode = ((lead + E4M3_BIAS) << 3) + mant
    ncode = np.minimum(ncode, 0x7E)                    # saturate to 448
    codes = np.where(big, ncode, codes)
    codes = np.where(a >= E4M3_MAX, 0x7E, codes)
    codes = codes.astype(np.int64) | np.where(np.signbit(x), 0x80, 0)
    codes = np.where(nan, 0x7F, codes)
    return codes.astype(np.uint8)
