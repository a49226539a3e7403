"""Small helpers for the tests: ulp distances and float bit views."""
import numpy as np


def f32_bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def ordered(x):
    """Map fp32 bit patterns to integers that order like the values, so the
    difference of two is their distance in ulps (+0 and -0 coincide)."""
    b = f32_bits(x).astype(np.int64)
    return np.where(b & 0x80000000, 0x80000000 - b, b)


def ulp_diff(a, b):
    return np.abs(ordered(a) - ordered(b))


def ordered16(h):
    """Same for 16-bit (bf16 or fp16) bit patterns."""
    b = np.ascontiguousarray(h, dtype=np.uint16).astype(np.int64)
    return np.where(b & 0x8000, 0x8000 - b, b)


def ulp16_diff(a, b):
    return np.abs(ordered16(a) - ordered16(b))


def same_or_both_nan16(a, b, nan_mask_bits=0x7F80, mant_mask=0x007F):
    a = np.asarray(a, dtype=np.uint16)
    b = np.asarray(b, dtype=np.uint16)
    an = ((a & nan_mask_bits) == nan_mask_bits) & ((a & mant_mask) != 0)
    bn = ((b & nan_mask_bits) == nan_mask_bits) & ((b & mant_mask) != 0)
    return np.where(an | bn, an & bn, a == b)


def rel_err(gpu, ref):
    """|gpu - ref| / max(|ref|, 2^-126) elementwise, in float64."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    return np.abs(g - r) / np.maximum(np.abs(r), 2.0 ** -126)


def rne_f32(v):
    """The binary32 value nearest the rational v (a Fraction or anything it
    converts), ties to even, normal range -- computed exactly, with no
    detour through double."""
    from fractions import Fraction
    v = Fraction(v)
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    unit = Fraction(2) ** (e - 23)            # the ulp of [2^e, 2^(e+1))
    m = a / unit                              # in [2^23, 2^24)
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * unit


def rint_even(v):
    """The integer nearest the rational v, ties to even."""
    from fractions import Fraction
    v = Fraction(v)
    lo = v.numerator // v.denominator
    rem = v - lo
    return lo + 1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1) else lo
