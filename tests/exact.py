"""Exact-arithmetic helpers for pinning the oracle (independent of oracle/).

bf16 rounding is checked here from its defining property -- the chosen bf16
value is a nearest one, and on a tie its last significand bit is 0 -- using
``fractions.Fraction`` so that no floating-point step is involved.
"""

from fractions import Fraction

import numpy as np

BF16_INF_MAG = 0x7F80


def bf16_mag_value(m):
    """Exact value of a non-negative bf16 magnitude pattern (0..0x7F80).
    The infinity pattern is given the value 2^128, the point where rounding
    overflows."""
    m = int(m)
    if m == BF16_INF_MAG:
        return Fraction(2) ** 128
    e, f = m >> 7, m & 0x7F
    if e == 0:
        return Fraction(f) * Fraction(2) ** -133
    return Fraction(128 + f) * Fraction(2) ** (e - 127 - 7)


def is_bf16_rne(v, bits):
    """True if bf16 pattern ``bits`` is the round-to-nearest-even of the exact
    rational ``v``."""
    bits = int(bits)
    sign, m = bits >> 15, bits & 0x7FFF
    if m > BF16_INF_MAG:
        return False  # NaN never is
    if v != 0 and (v < 0) != bool(sign):
        return False
    a = abs(v)
    d0 = abs(a - bf16_mag_value(m))
    cands = []
    if m > 0:
        cands.append(m - 1)
    if m < BF16_INF_MAG:
        cands.append(m + 1)
    for c in cands:
        dc = abs(a - bf16_mag_value(c))
        if dc < d0:
            return False
        if dc == d0 and (m & 1):
            return False
    return True


def exact_bf16_rne(v):
    """bf16 bits nearest (ties to even) to the exact rational v, found by
    checking the candidates around the float64 approximation."""
    approx = float(v)
    sgn = 0x8000 if v < 0 else 0
    # start from truncation of the float32 view of the approximation
    f32 = np.float32(abs(approx)) if abs(approx) < 3.5e38 else np.float32(np.inf)
    base = int(np.array([f32], dtype=np.float32).view(np.uint32)[0] >> 16)
    for m in range(max(0, base - 2), min(BF16_INF_MAG, base + 2) + 1):
        if is_bf16_rne(v if v != 0 else Fraction(0), sgn | m):
            return sgn | m
    raise AssertionError("no bf16 candidate found for %r" % (v,))


def f64_to_bf16_bits_intmath(x):
    """Independent fp64 -> bf16 RNE for NORMAL bf16 results, done with integer
    arithmetic on the fp64 bit pattern (round the 52-bit fraction at bit 45)."""
    x = np.asarray(x, dtype=np.float64)
    u = x.view(np.uint64).astype(np.uint64)
    sign = (u >> np.uint64(63)).astype(np.uint64)
    mag = u & np.uint64(0x7FFFFFFFFFFFFFFF)
    lsb = (mag >> np.uint64(45)) & np.uint64(1)
    rounded = (mag + np.uint64(0xFFFFFFFFFFF) + lsb) >> np.uint64(45)   # half-ulp minus 1, plus lsb: ties to even
    e64 = (rounded >> np.uint64(7)).astype(np.int64)
    frac = (rounded & np.uint64(0x7F)).astype(np.int64)
    e8 = e64 - 1023 + 127
    zero = mag == 0
    assert np.all(zero | ((e8 >= 1) & (e8 <= 254))), "outside the normal bf16 range"
    out = (sign.astype(np.int64) << 15) | (np.where(zero, 0, e8) << 7) | np.where(zero, 0, frac)
    return out.astype(np.uint16)
