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
