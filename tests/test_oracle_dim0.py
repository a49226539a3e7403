"""Pins of the oracle's per-parameter dim-0 sharding and its fp32 gradient
rows (CPU only).

"ZeRO and FSDP" (Zero to Frontier 10.3), FSDP section: FSDP2 stores each
parameter as a distributed tensor sharded along its first dimension and
packs a unit's shards into one buffer for each collective; with its mixed-
precision policy the gradient shards come out of a float32 reduce-scatter.
References: torch.chunk (the library routine that cuts a tensor along a
dimension), round trips, exact sums, and the already pinned 16-bit path."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import BF16, F32, tag
from synth.workloads import llama7b_numels

U = 2.0 ** -24


def _random_shapes(rng, k=12):
    shapes = []
    for _ in range(k):
        rows = int(rng.integers(0, 60))
        cols = int(rng.choice([1, 2, 3, 7, 16]))
        shapes.append((rows, cols))
    return shapes


@pytest.mark.parametrize("seed", range(20))
def test_segments_follow_torch_chunk(seed):
    rng = np.random.default_rng(seed)
    shapes = _random_shapes(rng)
    n_dp = int(rng.integers(1, 12))
    offs, chunk, n, s = oracle.dim0_layout(shapes, n_dp)
    assert n == sum(r * c for r, c in shapes)
    for rank in range(n_dp):
        segs = oracle.dim0_segments(shapes, n_dp, rank)
        held = {t: (toff, soff, ln) for t, toff, soff, ln in segs if t >= 0}
        for i, (rows, cols) in enumerate(shapes):
            pieces = torch.arange(rows * cols).reshape(rows, cols).chunk(n_dp, dim=0) \
                if rows else ()
            mine = pieces[rank].reshape(-1) if rank < len(pieces) else torch.empty(0)
            if mine.numel() == 0:
                assert i not in held
            else:
                toff, soff, ln = held[i]
                assert (toff, ln) == (int(mine[0]), mine.numel())
                assert soff == offs[i]
            # every rank's chunk has the same padded size
            full = pieces[0].numel() if rows else 0
            assert chunk[i] * cols == full
        # the pieces tile [0, S) in order
        pos = 0
        for _, _, soff, ln in segs:
            assert soff == pos
            pos += ln
        assert pos == s


@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("align", [1, 8])
def test_pack_then_unpack_rebuilds_every_tensor(seed, align):
    rng = np.random.default_rng(100 + seed)
    shapes = _random_shapes(rng, 9)
    n_dp = int(rng.integers(1, 9))
    tensors = [rng.standard_normal(r * c).astype(np.float32) + 1 for r, c in shapes]
    _, _, n, s = oracle.dim0_layout(shapes, n_dp, align)
    assert s % align == 0
    bufs = []
    for rank in range(n_dp):
        buf = np.full(s, np.nan, np.float32)
        for t, toff, soff, ln in oracle.dim0_segments(shapes, n_dp, rank, align):
            buf[soff:soff + ln] = 0.0 if t < 0 else tensors[t][toff:toff + ln]
        assert not np.isnan(buf).any()
        bufs.append(buf)
    back = [np.full(r * c, np.nan, np.float32) for r, c in shapes]
    for rank in range(n_dp):
        for t, toff, soff, ln in oracle.dim0_segments(shapes, n_dp, rank, align):
            if t >= 0:
                back[t][toff:toff + ln] = bufs[rank][soff:soff + ln]
    for a, b in zip(back, tensors):
        assert np.array_equal(a, b)
    # padding carries nothing: the packed buffers hold exactly N values
    assert sum(int(np.count_nonzero(b)) for b in bufs) == n


def _llama7b_shapes():
    d, ffn, vocab = 4096, 11008, 32000
    out = [(vocab, d)]
    for _ in range(32):
        out += [(d, d)] * 4 + [(ffn, d), (ffn, d), (d, ffn), (d, 1), (d, 1)]
    out += [(d, 1), (vocab, d)]
    return out


def test_llama7b_shapes_shard_evenly():
    shapes = _llama7b_shapes()
    assert [r * c for r, c in shapes] == llama7b_numels()
    for n_dp in (8, 64):
        _, _, n, s = oracle.dim0_layout(shapes, n_dp)
        assert n == 6_738_415_616 and s * n_dp == n  # every first dimension divides
    _, _, n, s = oracle.dim0_layout(shapes, 12)
    assert s * 12 > n  # 4096 / 12 and 32000 / 12 do not divide: padding


# ---- fp32 gradient rows -------------------------------------------------

def _rows32(n, length, sigma=1e-3, cfg=95):
    return np.stack([synth.fill_host(F32, 0, tag(synth.synth_const.BUF_GRAD, cfg, 0, 0, k), 0,
                                     length, sigma) for k in range(n)])


@pytest.mark.parametrize("n", [1, 3, 8])
def test_fp32_rows_equal_the_16bit_path_on_shared_values(n):
    """bf16 values widen exactly, so fp32 rows holding them must give the
    bf16 path's results bit for bit (reduce, accumulate, step, flags)."""
    length = 2000
    r16 = np.stack([synth.fill_host(BF16, 0, tag(synth.synth_const.BUF_GRAD, 96, 0, 0, k), 0,
                                    length, 1e-3) for k in range(n)])
    r16[n - 1, 7] = 0x7F80  # +inf in the last row
    r32 = oracle.bf16_to_f32(r16)
    outs = []
    for rows, gdt in ((r16, oracle.BF16), (r32, oracle.FP32)):
        acc = np.zeros(length, np.float32)
        ovf = np.zeros(1, np.uint32)
        ss = np.zeros(1, np.float64)
        oracle.reduce(rows, gdt, n, length, length, acc, 0, overflow=ovf)
        oracle.reduce(rows, gdt, n, length, length, acc, 1, sumsq=ss)
        w = synth.fill_host(F32, 0, tag(2, 96), 0, length, 0.02)
        m, v, wo = np.zeros(length, np.float32), np.zeros(length, np.float32), np.zeros(length, np.uint16)
        sovf = np.zeros(1, np.uint32)
        oracle.step(rows, gdt, n, length, length, w, m, v, wo, oracle.BF16, 1, overflow=sovf)
        outs.append((acc, ovf, w, m, v, wo, sovf))
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    assert outs[0][1][0] == 1 and outs[0][6][0] == 1


@pytest.mark.parametrize("n", [2, 8, 64])
def test_fp32_sum_within_bound_and_left_to_right(n):
    length = 1500
    rows = _rows32(n, length, sigma=1.0, cfg=97)
    acc = np.zeros(length, np.float32)
    oracle.reduce(rows, oracle.FP32, n, length, length, acc, 0)
    lr = rows[0].copy()
    for k in range(1, n):
        lr = (lr + rows[k]).astype(np.float32)
    assert np.array_equal(acc.view(np.uint32), lr.view(np.uint32))
    for j in range(0, length, 97):
        ex = sum(Fraction(float(rows[k, j])) for k in range(n))
        bound = Fraction((n - 1) * U) * sum(abs(Fraction(float(rows[k, j]))) for k in range(n))
        assert abs(Fraction(float(acc[j])) - ex) <= bound * Fraction(1000001, 1000000)


def test_fp32_rows_read_with_their_stride():
    """Row k starts at element k * ld (ld > len): the extra elements are
    never read."""
    n, length, ld = 4, 100, 130
    rows = _rows32(n, ld, cfg=98)
    rows[:, length:] = np.nan
    acc = np.zeros(length, np.float32)
    oracle.reduce(rows.reshape(-1), oracle.FP32, n, ld, length, acc, 0)
    want = rows[0, :length].copy()
    for k in range(1, n):
        want = (want + rows[k, :length]).astype(np.float32)
    assert np.array_equal(acc.view(np.uint32), want.view(np.uint32))
