"""Pins of the oracle's gradient reduce (the reduce-scatter's arithmetic).

"ZeRO and FSDP" (Zero to Frontier 10.3), "The idea, one stage at a time":
rank r receives the averaged gradient of shard r; a ring all-reduce is a
reduce-scatter followed by an all-gather.  The oracle sums the n 16-bit rows
in fp32, left to right; the average's 1/n is applied with the update.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from synth import BF16, F16, tag

U = 2.0 ** -24  # unit roundoff of fp32


def _rows(n, length, kind=BF16, sigma=1e-3, seed=0, thr=0, mul=1.0, cfg=90):
    return np.stack([synth.fill_host(kind, seed, tag(synth.synth_const.BUF_GRAD, cfg, 0, 0, k),
                                     0, length, sigma, thr, mul) for k in range(n)])


def _widen(rows, gdt):
    return oracle.f16_to_f32(rows) if gdt == oracle.FP16 else oracle.bf16_to_f32(rows)


@pytest.mark.parametrize("n", [1, 2, 3, 8, 64])
@pytest.mark.parametrize("gdt", [oracle.BF16, oracle.FP16])
def test_sum_within_recursive_summation_bound(n, gdt):
    length = 3000
    rows = _rows(n, length, BF16 if gdt == oracle.BF16 else F16,
                 sigma=1e-3 if gdt == oracle.BF16 else 65.536)
    acc = np.zeros(length, dtype=np.float32)
    oracle.reduce(rows, gdt, n, length, length, acc, 0)
    x = _widen(rows, gdt).astype(np.float64)
    exact = x.sum(axis=0)  # float64 sum of <= 64 short-mantissa values is exact here
    bound = (n - 1) * U * np.abs(x).sum(axis=0) * (1 + 1e-6)
    assert np.all(np.abs(acc.astype(np.float64) - exact) <= bound)
    if n == 1:
        assert np.array_equal(acc.view(np.uint32), x[0].astype(np.float32).view(np.uint32))


def test_sum_against_exact_fractions_tiny():
    rows = _rows(5, 16, sigma=1.0, cfg=91)
    acc = np.zeros(16, dtype=np.float32)
    oracle.reduce(rows, oracle.BF16, 5, 16, 16, acc, 0)
    x = oracle.bf16_to_f32(rows)
    for j in range(16):
        ex = sum(Fraction(float(x[k, j])) for k in range(5))
        bound = Fraction(4 * U) * sum(abs(Fraction(float(x[k, j]))) for k in range(5))
        assert abs(Fraction(float(acc[j])) - ex) <= bound
    # left-to-right order, exactly: ((x0 + x1) + x2) + ...
    lr = x[0].copy()
    for k in range(1, 5):
        lr = (lr + x[k]).astype(np.float32)
    assert np.array_equal(acc.view(np.uint32), lr.view(np.uint32))


def test_row_stride_and_offset_are_honoured():
    # rows of a wider [n][ld] slab, read at an offset: only elements
    # [off, off + len) of each row may contribute
    n, ld, off, length = 4, 1000, 123, 500
    slab = _rows(n, ld, cfg=92)
    acc = np.zeros(length, dtype=np.float32)
    sub = np.ascontiguousarray(slab.reshape(-1)[off:])
    oracle.reduce(sub, oracle.BF16, n, ld, length, acc, 0)
    ref = np.zeros(length, dtype=np.float32)
    oracle.reduce(np.ascontiguousarray(slab[:, off:off + length]), oracle.BF16, n, length,
                  length, ref, 0)
    assert np.array_equal(acc.view(np.uint32), ref.view(np.uint32))


def test_reduce_scatter_then_all_gather_equals_all_reduce():
    n_dp, numels = 4, [1000, 37, 2999]
    _, n, n_pad, s = oracle.flatten_layout(numels, n_dp)
    full = _rows(n_dp, n_pad, cfg=93)
    full[:, n:] = 0  # padding gradients are zero
    ar = np.zeros(n_pad, dtype=np.float32)
    oracle.reduce(full, oracle.BF16, n_dp, n_pad, n_pad, ar, 0)  # all-reduce (sum)
    gathered = np.zeros(n_pad, dtype=np.float32)
    for r in range(n_dp):  # reduce-scatter: shard r of every rank's gradient
        piece = np.zeros(s, dtype=np.float32)
        sub = np.ascontiguousarray(full.reshape(-1)[r * s:])
        oracle.reduce(sub, oracle.BF16, n_dp, n_pad, s, piece, 0)
        gathered[r * s:(r + 1) * s] = piece  # all-gather
    assert np.array_equal(gathered.view(np.uint32), ar.view(np.uint32))
    assert np.all(ar[n:] == 0)


def test_accumulate_adds_partial_sums():
    n, length = 8, 2000
    mbs = [_rows(n, length, F16, sigma=65.536, cfg=94 + i) for i in range(4)]
    acc = np.full(length, 7.0, dtype=np.float32)  # stale contents are overwritten
    for i, rows in enumerate(mbs):
        oracle.reduce(rows, oracle.FP16, n, length, length, acc, int(i > 0))
    parts = []
    for rows in mbs:
        p = np.zeros(length, dtype=np.float32)
        oracle.reduce(rows, oracle.FP16, n, length, length, p, 0)
        parts.append(p)
    ref = parts[0]
    for p in parts[1:]:
        ref = (ref + p).astype(np.float32)
    assert np.array_equal(acc.view(np.uint32), ref.view(np.uint32))
    x = np.stack([_widen(r, oracle.FP16) for r in mbs]).astype(np.float64)
    exact = x.sum(axis=(0, 1))
    bound = (4 * n) * U * np.abs(x).sum(axis=(0, 1))
    assert np.all(np.abs(acc - exact) <= bound)


@pytest.mark.parametrize("pos", [0, 999, 500])
@pytest.mark.parametrize("bad", [0x7C00, 0xFC00, 0x7E00])
def test_overflow_flag_on_nonfinite_input(pos, bad):
    rows = _rows(3, 1000, F16, sigma=65.536, cfg=97)
    flag = np.zeros(1, dtype=np.uint32)
    acc = np.zeros(1000, dtype=np.float32)
    oracle.reduce(rows, oracle.FP16, 3, 1000, 1000, acc, 0, overflow=flag)
    assert flag[0] == 0
    rows[1, pos] = bad
    oracle.reduce(rows, oracle.FP16, 3, 1000, 1000, acc, 0, overflow=flag)
    assert flag[0] == 1


def test_sum_of_negative_zero_rows_keeps_the_sign():
    """The sum starts from row 0 itself (not from +0), so rows of -0 add up
    to -0 under round-to-nearest, and a single row comes back unchanged."""
    rows = np.full((3, 16), 0x8000, np.uint16)  # bf16 -0
    acc = np.zeros(16, np.float32)
    oracle.reduce(rows, oracle.BF16, 3, 16, 16, acc, 0)
    assert np.all(acc.view(np.uint32) == 0x80000000)


def test_sumsq_is_that_of_the_accumulated_gradient():
    """With accumulation, the sum of squares is over the accumulator after
    the call (the gradient the update will use), not over the call's own
    partial sum."""
    n, length = 4, 3000
    acc = np.zeros(length, dtype=np.float32)
    oracle.reduce(_rows(n, length, cfg=99), oracle.BF16, n, length, length, acc, 0)
    ss = np.zeros(1, dtype=np.float64)
    oracle.reduce(_rows(n, length, cfg=100), oracle.BF16, n, length, length, acc, 1, sumsq=ss)
    ref = np.sum(acc.astype(np.float64) ** 2)
    assert abs(ss[0] - ref) <= 1e-12 * ref


def test_sumsq_matches_float64():
    rows = _rows(8, 4096, cfg=98)
    acc = np.zeros(4096, dtype=np.float32)
    ss = np.zeros(1, dtype=np.float64)
    oracle.reduce(rows, oracle.BF16, 8, 4096, 4096, acc, 0, sumsq=ss)
    ref = np.sum(acc.astype(np.float64) ** 2)
    assert abs(ss[0] - ref) <= 1e-12 * ref
