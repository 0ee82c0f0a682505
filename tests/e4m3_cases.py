"""Hand-worked e4m3fn cases shared by the CPU oracle pins and the GPU append test.

OCP e4m3fn: bias 7, 3 mantissa bits, largest finite 448 (code 0x7E),
subnormals m * 2^-9. Round to nearest, a tie between two neighbouring codes
going to the one with the even mantissa (the even code).

TIE_VALUES, with their codes worked out by hand:
  448            exactly the largest code                     0x7E
  -448                                                        0xFE
  440            halfway between 432 (0x7D) and 448 (0x7E)    0x7E (even)
  248            halfway between 240 (0x77) and 256 (0x78)    0x78 (even)
  1.0625         halfway between 1 (0x38) and 1.125 (0x39)    0x38 (even)
  1.1875         halfway between 1.125 (0x39) and 1.25 (0x3A) 0x3A (even)
  -1.0625                                                     0xB8
  2^-10          halfway between 0 and 2^-9 (0x01)            0x00 (even)
  3 * 2^-10      halfway between 2^-9 (0x01) and 2^-8 (0x02)  0x02 (even)
  5 * 2^-10      halfway between 2^-8 (0x02) and 3*2^-9 (0x03) 0x02 (even)
  -3 * 2^-10                                                  0x82
  2^-11          below half of 2^-9                           0x00
  15 * 2^-10     halfway between 7 * 2^-9 (0x07) and 2^-6 (0x08, the first
                 normal code)                                 0x08 (even)
  0                                                           0x00
  1                                                           0x38
  0.5                                                         0x30
"""

import numpy as np

TIE_VALUES = [448.0, -448.0, 440.0, 248.0, 1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10,
              5 * 2.0 ** -10, -3 * 2.0 ** -10, 2.0 ** -11, 15 * 2.0 ** -10, 0.0, 1.0, 0.5]

TIE_CODES = np.array([0x7E, 0xFE, 0x7E, 0x78, 0x38, 0x3A, 0xB8, 0x00, 0x02, 0x02, 0x82, 0x00,
                      0x08, 0x00, 0x38, 0x30], dtype=np.uint8)


def nearest_code_brute(y, decode):
    """e4m3 code of each real y by exhaustive search: the finite code whose
    value is nearest |y| (0x7E for anything beyond 448), the even one of two
    equally near neighbours, with y's sign bit. `decode` maps codes to
    values (only the 127 non-negative finite codes are searched)."""
    y = np.asarray(y, dtype=np.float64)
    codes = np.arange(0x7F)                                   # +0 .. 448
    mags = decode(codes.astype(np.uint8))
    a = np.abs(y.reshape(-1))
    d = np.abs(mags[None, :] - a[:, None])
    near = d == d.min(axis=1, keepdims=True)
    even = near & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), near.argmax(axis=1))
    pick = pick | np.where(np.signbit(y.reshape(-1)), 0x80, 0)
    return pick.reshape(y.shape).astype(np.uint8)
