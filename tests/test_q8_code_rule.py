"""The device quantizer's shortcut gives the oracle's codes (CPU only).

The oracle codes an element as rint(fl(x / s)) with s = fl(absmax / 127)
(one correctly rounded division per element).  The device kernel forms
y = fl(x * r) with the block's r = fl(127 / absmax) and divides only where y
lies within 2^-14 of a half-integer, or where s is subnormal; its comment
gives the error bound that makes rint(y) equal to rint(fl(x / s))
everywhere else.  These tests restate that rule in NumPy binary32 (IEEE
operations, round to nearest even, subnormals kept) and check it against
the oracle element by element where the two readings could part: every
half-integer code boundary of many block scales, dense in ulps around each
one, the blocks the oracle's pins found by search, subnormal scales and
random blocks.  They also measure the bound itself.  The same adversarial
blocks go through the device kernel in the GPU tests."""
import numpy as np
import pytest

import oracle

B = oracle.Q8_BLOCK
F = np.float32
BAND = F(0.5 - 2.0 ** -14)


def kernel_rule(x, amax):
    """The device's codes for values x of a block whose absmax is amax."""
    amax = F(amax)
    s = amax / F(127.0)
    if not (s > 0) or np.isinf(s):
        return np.zeros(x.shape, np.int8)
    with np.errstate(over="ignore", invalid="ignore"):
        r = F(127.0) / amax
        y = (x * r).astype(F)
        k = np.rint(y)
        near = np.abs((y - k).astype(F)) >= BAND
        if s < F(2.0 ** -126):
            near[:] = True
        k = np.where(near, np.rint((x / s).astype(F)), k)
    return np.clip(k, -127, 127).astype(np.int8)


def neighbourhoods(amax, ulps):
    """For every half-integer h in (-127, 127): the binary32 values within
    `ulps` ulps of h * s (clipped to the block), so that each boundary
    between two codes is crossed element by element."""
    amax = F(amax)
    s = amax / F(127.0)
    h = (np.arange(-127, 127, dtype=np.float64) + 0.5)
    centre = (h * float(s)).astype(F)
    bits = centre.view(np.int32).astype(np.int64)
    offs = np.arange(-ulps, ulps + 1, dtype=np.int64)
    # walk in ulps through the integer representation (same sign side)
    x = (bits[:, None] + offs[None, :]).astype(np.int32).view(F).reshape(-1)
    x = x[np.isfinite(x) & (np.abs(x) <= amax)]
    return np.concatenate([[amax], x]).astype(F)


def check(x, amax):
    """x (all |x| <= amax) as blocks of the oracle that each open with amax,
    so that every block's absmax is amax."""
    amax = F(amax)
    n = -(-x.size // (B - 1))
    blocks = np.zeros((n, B), F)
    blocks[:, 0] = amax
    flat = np.zeros(n * (B - 1), F)
    flat[:x.size] = x
    blocks[:, 1:] = flat.reshape(n, B - 1)
    blocks[-1, 1 + x.size - (n - 1) * (B - 1):] = amax    # no zero filler in the last block
    q_ref, s_ref = oracle.q8_quantize(blocks.reshape(-1), oracle.FP32)
    assert np.all(s_ref == amax / F(127.0))
    x = blocks.reshape(-1)
    got = kernel_rule(x, amax)
    bad = np.nonzero(got != q_ref)[0]
    assert bad.size == 0, (float(amax), x[bad[:5]], got[bad[:5]], q_ref[bad[:5]])
    return x.size


def _scales(seed, n):
    rng = np.random.default_rng(seed)
    amax = rng.uniform(0.5, 2.0, size=n) * np.exp2(rng.integers(-100, 100, size=n))
    return amax.astype(F)


@pytest.mark.parametrize("seed", range(6))
def test_every_code_boundary_of_random_scales(seed):
    total = 0
    for amax in _scales(seed, 40):
        total += check(neighbourhoods(amax, 48), amax)
    assert total > 40 * 254 * 90


def test_scales_that_make_the_shortcut_exact_or_tight():
    """absmax = 127 * 2^k (s a power of two, r exact), absmax just below and
    above powers of two, and the largest finite absmax."""
    cases = [F(127.0), F(127.0 * 2.0 ** -60), F(127.0 * 2.0 ** 40), F(1.0), F(2.0),
             np.nextafter(F(1.0), F(0.0)), np.nextafter(F(2.0), F(4.0)),
             np.nextafter(F(128.0), F(0.0)), F(np.finfo(F).max), F(3.4e38 / 1.5)]
    for amax in cases:
        check(neighbourhoods(amax, 64), amax)


def test_blocks_found_by_the_oracles_search():
    from tests.test_oracle_q8 import _search_blocks_telling_the_readings_apart
    found = _search_blocks_telling_the_readings_apart(7, want=32)
    assert len(found) >= 16
    for amax, xv in found:
        check(np.array([amax, xv], F), amax)


def test_subnormal_and_tiny_scales():
    """s subnormal: the shortcut is off and every code is a division; s = 0:
    all codes zero; the smallest normal s."""
    tiny = F(2.0 ** -149)
    for amax in [F(1e-38), F(2.0 ** -126) * F(127.0), F(2.0 ** -126) * F(126.9),
                 F(64) * tiny, F(63) * tiny, F(1e-40), F(2.0 ** -126)]:
        rng = np.random.default_rng(int(amax.view(np.int32)))
        x = (rng.uniform(-1, 1, size=4 * B) * float(amax)).astype(F)
        x = np.concatenate([[amax], x, neighbourhoods(amax, 8)]).astype(F)
        check(x, amax)


def test_random_blocks():
    rng = np.random.default_rng(3)
    for _ in range(300):
        x = (rng.standard_normal(B) * 10.0 ** rng.uniform(-30, 30)).astype(F)
        amax = np.abs(x).max()
        check(x, amax)


def test_the_bound_behind_the_band():
    """Where s is normal, y = fl(x * r) stays within 2.28e-5 of the exact
    x / s and the binary32 quotient within 2^-18 of it: their distance never
    reaches the band's 2^-14, measured over every boundary neighbourhood."""
    from fractions import Fraction
    worst = 0.0
    for amax in _scales(99, 12):
        x = neighbourhoods(amax, 16)
        s = F(amax) / F(127.0)
        r = F(127.0) / F(amax)
        y = (x * r).astype(F).astype(np.float64)
        q = (x / s).astype(F).astype(np.float64)
        worst = max(worst, float(np.max(np.abs(y - q))))
        # spot-check the exact quotient on a few elements
        for xv in x[:: max(1, x.size // 20)]:
            ex = Fraction(float(xv)) / Fraction(float(s))
            assert abs(float(Fraction(float(F(xv * r))) - ex)) < 2.28e-5
    assert worst < 2.28e-5 + 2.0 ** -18 < 2.0 ** -14
