"""Pins of the oracle's 8-bit blockwise quantizer and quantized step (CPU).

The pages name ZeRO++'s 8-bit weight all-gather and quantized gradient
reduce-scatter ("ZeRO and FSDP", FSDP section; "ZeRO: How DeepSpeed Made
Trillion-Parameter Training Practical"; "ZeRO Optimizer, in depth",
"Offload and ZeRO++") but define no quantizer.  PARITY UNPINNED against the
pages: these tests pin the stated quantizer (symmetric, one fp32 scale per
256-element block, s = absmax / 127, q = rint(x / s): the value measured in
units of the stored scale) to its mathematical properties and to
hand-worked examples."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from synth import F32, tag
from tests.util import rint_even, rne_f32

U = 2.0 ** -24
B = oracle.Q8_BLOCK


def _x(n, seed, sigma=1.0):
    return synth.fill_host(F32, seed, tag(5, 150), 0, n, sigma,
                           synth.synth_const.outlier_threshold(0.01), 100.0)


def test_hand_worked_block():
    # absmax 1: s = fl(1/127) = 2113665 * 2^-28, a little below 1/127.
    # 0.5 / s = 63.50000024 exactly, whose nearest binary32 is 63.5 (ulp
    # 2^-18): the code is rint(63.5) = 64, a tie to even; -0.25 / s rounds to
    # -31.75 -> -32, 0.1 / s to 12.7 -> 13, 0.0236 / s to 2.9972 -> 3
    x = np.array([1.0, 0.5, -0.25, 0.1, 0.0236, 0.0], np.float32)
    q, s = oracle.q8_quantize(x, oracle.FP32)
    assert s[0] == np.float32(1.0) / np.float32(127.0)
    assert Fraction(float(s[0])) == Fraction(2113665, 2 ** 28)
    assert q.tolist() == [127, 64, -32, 13, 3, 0]
    # absmax 127 makes s exactly 1: the codes are the values rounded,
    # ties to the even code (62.5 -> 62, -0.5 -> 0, 2.5 -> 2, -3.5 -> -4)
    x = np.array([127.0, 62.5, -0.5, 1.5, 2.5, -3.5, -127.0], np.float32)
    q, s = oracle.q8_quantize(x, oracle.FP32)
    assert s[0] == 1.0 and q.tolist() == [127, 62, 0, 2, 2, -4, -127]


@pytest.mark.parametrize("n", [1, 255, 256, 257, 4096, 10_001])
def test_codes_range_absmax_and_rounding_bound(n):
    x = _x(n, n)
    q, s = oracle.q8_quantize(x, oracle.FP32)
    assert s.size == (n + B - 1) // B
    assert q.min() >= -127 and q.max() <= 127
    for b in range(s.size):
        blk, qb = x[b * B:(b + 1) * B], q[b * B:(b + 1) * B]
        amax = np.abs(blk).max()
        assert s[b] == np.float32(amax) / np.float32(127.0)
        if amax > 0:
            assert np.abs(qb).max() == 127
            assert qb[np.argmax(np.abs(blk))] == np.sign(blk[np.argmax(np.abs(blk))]) * 127
        err = np.abs(blk.astype(np.float64) - qb.astype(np.float64) * float(s[b]))
        assert np.all(err <= float(s[b]) * (0.5 + 128 * U))


@pytest.mark.parametrize("k", [-20, -3, 1, 7, 30])
def test_power_of_two_scaling_is_exact(k):
    x = _x(3000, 7, sigma=1e-2)
    q, s = oracle.q8_quantize(x, oracle.FP32)
    q2, s2 = oracle.q8_quantize((x * np.float32(2.0 ** k)).astype(np.float32), oracle.FP32)
    assert np.array_equal(q, q2)
    assert np.array_equal(s2, (s * np.float32(2.0 ** k)).astype(np.float32))


def test_sign_symmetry():
    x = _x(5000, 8)
    q, s = oracle.q8_quantize(x, oracle.FP32)
    qn, sn = oracle.q8_quantize(-x, oracle.FP32)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)


def test_zero_and_nonfinite_blocks():
    x = _x(4 * B, 9)
    x[:B] = 0.0
    x[B + 17] = np.inf
    x[2 * B + 5] = np.nan
    q, s = oracle.q8_quantize(x, oracle.FP32)
    assert s[0] == 0 and not q[:B].any()
    assert np.isinf(s[1]) and not q[B:2 * B].any()
    assert np.isnan(s[2]) and not q[2 * B:3 * B].any()
    y = oracle.q8_dequantize(q, s)
    assert np.all(y[:B] == 0) and np.all(np.isnan(y[B:3 * B])) and np.all(np.isfinite(y[3 * B:]))


def test_tiny_blocks_code_until_the_scale_underflows_to_zero():
    """Codes need only a non-zero finite scale: a block of subnormal-range
    magnitudes still codes (its scale a subnormal, the largest element
    +-127), and only a block whose absmax / 127 rounds to zero (absmax at
    most 63 times the smallest subnormal) codes as zeros."""
    tiny = np.float32(2.0 ** -149)
    x = np.zeros(3 * B, np.float32)
    x[:B] = np.float32(1e-38) * np.sign(_x(B, 11))       # s subnormal
    x[B:2 * B] = np.float32(64) * tiny * np.sign(_x(B, 12))   # s = the smallest subnormal
    x[2 * B:] = np.float32(63) * tiny * np.sign(_x(B, 13))    # s = 0
    q, s = oracle.q8_quantize(x, oracle.FP32)
    assert 0 < s[0] < np.float32(2.0 ** -126) and np.abs(q[:B]).max() == 127
    assert s[1] == tiny
    # 64 * 2^-149 / 2^-149 = 64: the block's codes are +-64, not +-127,
    # because the scale itself is rounded (64/127 of a subnormal step)
    assert np.abs(q[B:2 * B]).max() == 64
    assert s[2] == 0 and not q[2 * B:].any()


def test_bf16_input_equals_its_fp32_widening():
    h = synth.fill_host(synth.BF16, 1, tag(5, 151), 0, 3001, 1e-3)
    q1, s1 = oracle.q8_quantize(h, oracle.BF16)
    q2, s2 = oracle.q8_quantize(oracle.bf16_to_f32(h), oracle.FP32)
    assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


def test_dequantize_16bit_is_the_rounded_fp32_value():
    x = _x(2000, 10)
    q, s = oracle.q8_quantize(x, oracle.FP32)
    y32 = oracle.q8_dequantize(q, s, oracle.FP32)
    assert np.array_equal(y32, (q.astype(np.float32) * np.repeat(s, B)[:q.size]).astype(np.float32))
    assert np.array_equal(oracle.q8_dequantize(q, s, oracle.BF16), oracle.f32_to_bf16(y32))
    assert np.array_equal(oracle.q8_dequantize(q, s, oracle.FP16), oracle.f32_to_f16(y32))


@pytest.mark.parametrize("n_dp", [1, 3, 8])
@pytest.mark.parametrize("scale_pad", [0, 3])
def test_quantized_step_is_dequantize_step_quantize(n_dp, scale_pad):
    """ora_step_q8 = dequantize each row to fp32, the fp32-row step (pinned
    elsewhere), then quantize the new master -- bit for bit.  With scale_pad
    the scale rows are wider than the code rows need (sld > ld / B), their
    padding a huge value that a wrong scale stride would pick up."""
    length, ld = 3 * B + 77, 4 * B
    sld = ld // B + scale_pad
    rows = np.stack([_x(ld, 20 + k, 1e-3) for k in range(n_dp)])
    qs = [oracle.q8_quantize(rows[k], oracle.FP32) for k in range(n_dp)]
    gq = np.concatenate([q for q, _ in qs])
    gs = np.full((n_dp, sld), 1e30, np.float32)
    for k, (_, s) in enumerate(qs):
        gs[k, :s.size] = s
    gs = gs.reshape(-1)
    w0 = _x(length, 30, 0.02)
    hp = dict(lr=1e-3, weight_decay=0.1)
    w, m, v = w0.copy(), np.zeros(length, np.float32), np.zeros(length, np.float32)
    wq = np.zeros(length, np.int8)
    ws = np.zeros(oracle.q8_blocks(length), np.float32)
    ss = np.zeros(1)
    oracle.step_q8(gq, gs, n_dp, ld, sld, length, w, m, v, wq, ws, 1, sumsq=ss, **hp)
    deq = np.stack([oracle.q8_dequantize(q, s) for q, s in qs])
    w2, m2, v2 = w0.copy(), np.zeros(length, np.float32), np.zeros(length, np.float32)
    wo = np.zeros(length, np.uint16)
    ss2 = np.zeros(1)
    oracle.step(deq.reshape(-1), oracle.FP32, n_dp, ld, length, w2, m2, v2, wo, oracle.BF16, 1,
                sumsq=ss2, **hp)
    for a, b in ((w, w2), (m, m2), (v, v2)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    q3, s3 = oracle.q8_quantize(w2, oracle.FP32)
    assert np.array_equal(wq, q3) and np.array_equal(ws.view(np.uint32), s3.view(np.uint32))
    assert ss[0] == ss2[0]


def _search_blocks_telling_the_readings_apart(seed, want=8):
    """(absmax, x) pairs whose code differs between rint(x / s) and
    rint(x * (127 / absmax)): elements within a few ulps of half-integer
    codes, the only place where the two can disagree."""
    rng = np.random.default_rng(seed)
    found = []
    for _ in range(400):
        amax = np.float32(rng.uniform(0.5, 2.0))
        s = amax / np.float32(127.0)
        k = rng.integers(-126, 127, size=4096).astype(np.float32)
        x = ((k + np.float32(0.5)) * s).astype(np.float32)
        x = x + rng.integers(-2, 3, size=x.size).astype(np.float32) * np.spacing(x)
        x = np.clip(x, -amax, amax).astype(np.float32)
        by_r = np.rint(x * (np.float32(127.0) / amax))
        by_s = np.rint(x / s)
        hit = np.nonzero(by_r != by_s)[0]
        if hit.size:
            found.append((amax, x[hit[0]]))
        if len(found) >= want:
            break
    return found


def test_codes_are_the_value_divided_by_the_stored_scale():
    """Pins q = rint(fl(x / s)), s = fl(absmax / 127), against the other
    plausible form, rint(fl(x * fl(127 / absmax))): blocks whose elements
    round differently under the two are found by search, and the expected
    code of each is derived in exact rational arithmetic with explicit
    round-to-nearest-even to binary32 at each operation."""
    found = _search_blocks_telling_the_readings_apart(7)
    assert len(found) >= 6
    for amax, xv in found:
        blk = np.array([amax, xv], np.float32)
        q, sc = oracle.q8_quantize(blk, oracle.FP32)
        s_ex = rne_f32(Fraction(float(amax)) / Fraction(127))
        want = rint_even(rne_f32(Fraction(float(xv)) / s_ex))
        r = rne_f32(Fraction(127) / Fraction(float(amax)))
        other = rint_even(rne_f32(Fraction(float(xv)) * r))
        assert want != other                      # the case tells the readings apart
        assert int(q[1]) == want and int(q[0]) == 127
        assert Fraction(float(sc[0])) == s_ex     # the stored scale is absmax / 127


def test_the_quotient_is_rounded_to_binary32_before_the_code():
    """The code rounds the binary32 quotient, not the exact one: where the
    exact x / s lies less than half an ulp from a half-integer k + 1/2, the
    binary32 quotient is k + 1/2 itself, a tie that goes to the even code,
    while the exact quotient would round to its nearer side.  Cases where
    the two differ are found by search over scales; each is derived in exact
    rational arithmetic."""
    rng = np.random.default_rng(11)
    cases = 0
    for _ in range(20000):
        amax = np.float32(rng.uniform(0.5, 2.0))
        s = amax / np.float32(127.0)
        k = int(rng.integers(0, 126))
        x = np.float32((k + 0.5) * float(s))
        if not x <= amax:
            continue
        exact = Fraction(float(x)) / Fraction(float(s))
        rounded = rne_f32(exact)
        if rounded != Fraction(2 * k + 1, 2) or exact == rounded:
            continue
        nearest = int(exact + Fraction(1, 2))     # exact > 0, not a tie
        want = rint_even(rounded)
        if nearest == want:
            continue                              # both roundings agree here
        q, _ = oracle.q8_quantize(np.array([amax, x], np.float32), oracle.FP32)
        assert int(q[1]) == want
        cases += 1
        if cases >= 4:
            break
    assert cases >= 4
