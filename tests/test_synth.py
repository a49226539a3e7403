"""The seeded input generator: deterministic, random access, the stated
distributions.  (It draws inputs only; the optimizer's arithmetic is pinned
elsewhere.)"""
import numpy as np

import oracle
import synth
from synth import BF16, F16, F32, tag


def test_fill_and_gather_agree_and_repeat():
    a = synth.fill_host(F32, 7, tag(2, 1), 1000, 50000, 0.02)
    b = synth.fill_host(F32, 7, tag(2, 1), 1000, 50000, 0.02, nthreads=1)
    assert np.array_equal(a, b)
    idx = np.array([1000, 1001, 25000, 50999])
    g = synth.gather_host(F32, 7, tag(2, 1), idx, 0.02)
    assert np.array_equal(g, a[idx - 1000])
    c = synth.fill_host(F32, 8, tag(2, 1), 1000, 50000, 0.02)
    assert not np.array_equal(a, c)


def test_distribution_and_outliers():
    n = 2_000_000
    x = synth.fill_host(F32, 0, tag(1), 0, n, 1e-3)
    assert abs(x.std() / 1e-3 - 1) < 0.01 and abs(x.mean()) < 1e-5
    thr = synth.outlier_threshold(0.01)
    y = synth.fill_host(F32, 0, tag(1), 0, n, 1e-3, thr, 100.0)
    rate = np.mean(y != x)
    assert abs(rate - 0.01) < 0.001
    assert np.allclose(y[y != x], 100.0 * x[y != x], rtol=1e-6)


def test_16bit_draws_truncate_the_float_draw():
    f = synth.fill_host(F32, 3, tag(1, 4), 0, 100000, 65.536)
    h = synth.fill_host(F16, 3, tag(1, 4), 0, 100000, 65.536)
    b = synth.fill_host(BF16, 3, tag(1, 4), 0, 100000, 65.536)
    hf = oracle.f16_to_f32(h)
    bf = oracle.bf16_to_f32(b)
    assert np.all(np.abs(hf) <= np.abs(f)) and np.all(np.abs(bf) <= np.abs(f))
    assert np.all(np.abs(f - hf) <= np.abs(f) * 2.0 ** -10 + 2.0 ** -24)
    assert np.all(np.abs(f - bf) <= np.abs(f) * 2.0 ** -7)
    assert np.all(np.isfinite(hf))
