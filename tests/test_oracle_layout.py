"""Pins of the oracle's flatten + shard layout (CPU only).

"ZeRO and FSDP" (Zero to Frontier 10.3), "The idea, one stage at a time":
one flat vector of N parameters, n_dp equal contiguous shards, rank r owns
shard r.  "A sharded Adam step" describes the shards as numpy.array_split
pieces; both readings agree whenever n_dp divides N.
"""
import json
import os

import numpy as np
import pytest

import oracle
from synth.workloads import gpt2xl_numels, llama7b_numels

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_tiny_workload_printed_sizes():
    g = json.load(open(os.path.join(GOLD, "tiny_layout.json")))
    offs, n, n_pad, s = oracle.flatten_layout(g["numels"], g["n_dp"], g["align"])
    assert (n, n_pad, s) == (g["n"], g["n_pad"], g["shard"])
    segs = oracle.shard_segments(g["numels"], g["n_dp"], g["rank"], g["align"])
    assert segs == [(0, g["slot_begin"], 0, g["slot_end"] - g["slot_begin"])]


@pytest.mark.parametrize("seed", range(6))
def test_equal_shards_match_numpy_array_split(seed):
    rng = np.random.default_rng(seed)
    n_dp = int(rng.integers(1, 17))
    n = n_dp * int(rng.integers(0, 5000))
    _, nn, n_pad, s = oracle.flatten_layout([n], n_dp)
    assert nn == n and n_pad == n
    pieces = np.array_split(np.arange(n), n_dp)
    for r, p in enumerate(pieces):
        assert len(p) == s
        if len(p):
            assert p[0] == r * s and p[-1] == r * s + s - 1
        assert oracle.array_split_start(n, n_dp, r) == (p[0] if len(p) else r * s)


@pytest.mark.parametrize("n,parts", [(10, 3), (7, 7), (5, 8), (0, 4), (1001, 16)])
def test_array_split_start_matches_numpy(n, parts):
    pieces = np.array_split(np.arange(n), parts)
    starts = np.cumsum([0] + [len(p) for p in pieces])[:-1]
    assert [oracle.array_split_start(n, parts, i) for i in range(parts)] == list(starts)


def _brute_owner(numels, n_pad):
    """For every flat index: (tensor, offset in tensor), or (-1, k) for padding."""
    out = []
    for t, k in enumerate(numels):
        out += [(t, i) for i in range(k)]
    n = len(out)
    out += [(-1, i) for i in range(n_pad - n)]
    return out


@pytest.mark.parametrize("seed", range(20))
def test_segments_tile_each_shard_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    numels = [int(x) for x in rng.integers(0, 9, size=int(rng.integers(0, 7)))]
    n_dp = int(rng.integers(1, 6))
    align = int(rng.choice([1, 2, 8]))
    offs, n, n_pad, s = oracle.flatten_layout(numels, n_dp, align)
    assert n == sum(numels)
    assert list(offs) == list(np.cumsum([0] + numels)[:-1])
    assert s % align == 0 and n_pad == n_dp * s and n_pad >= n
    assert n_pad - n < n_dp * align  # no more padding than needed
    owner = _brute_owner(numels, n_pad)
    for r in range(n_dp):
        seen = []
        for (t, toff, soff, ln) in oracle.shard_segments(numels, n_dp, r, align):
            assert ln > 0
            for i in range(ln):
                assert owner[r * s + soff + i] == (t, toff + i)
                seen.append(soff + i)
        assert seen == list(range(s))  # contiguous, in order, exactly the shard


def test_parameter_list_totals():
    # "~6.74e9" Llama-shaped 7B and "~1.56e9" GPT-2-XL-shaped parameter lists
    n7 = sum(llama7b_numels())
    ng = sum(gpt2xl_numels())
    assert float(f"{n7:.3g}") == 6.74e9
    assert float(f"{ng:.3g}") == 1.56e9
    assert len(llama7b_numels()) == 1 + 32 * 9 + 2
    # the one-rank shard sizes, "~842M" at n_dp = 8 and "~105M" at n_dp = 64
    s8 = oracle.flatten_layout(llama7b_numels(), 8)[3]
    s64 = oracle.flatten_layout(llama7b_numels(), 64)[3]
    assert round(s8 / 1e6) == 842 and round(s64 / 1e6) == 105
    assert s8 * 8 == n7 and s64 * 64 == n7  # n_dp divides N: no padding


def test_large_segment_map_is_consistent():
    numels = llama7b_numels()
    offs, n, n_pad, s = oracle.flatten_layout(numels, 8)
    for r in range(8):
        segs = oracle.shard_segments(numels, 8, r)
        assert sum(q[3] for q in segs) == s
        pos = 0
        for (t, toff, soff, ln) in segs:
            assert soff == pos
            assert 0 <= toff and toff + ln <= numels[t]
            assert offs[t] + toff == r * s + soff
            pos += ln


@pytest.mark.parametrize("args", [([4], 0, 1), ([4], 2, 0), ([-1], 2, 1)])
def test_invalid_layout_rejected(args):
    with pytest.raises(ValueError):
        oracle.flatten_layout(*args)


def test_empty_vector():
    assert oracle.flatten_layout([], 4)[1:] == (0, 0, 0)
    assert oracle.shard_segments([], 4, 3) == []


def test_sizes_beyond_int64_are_rejected():
    """A layout whose N or N_pad would not fit int64 is rejected rather than
    wrapped; the largest that fit come out exact."""
    big = (1 << 63) - 1
    for nums, n_dp, align in [([big, 1], 1, 1), ([big // 2, big // 2 + 2], 1, 1),
                              ([big - 5], 4, 8), ([1], 1 << 30, big // 4)]:
        with pytest.raises(ValueError):
            oracle.flatten_layout(nums, n_dp, align)
    _, n, n_pad, s = oracle.flatten_layout([big], 1, 1)
    assert n == n_pad == s == big
    _, n, n_pad, s = oracle.flatten_layout([1 << 62], 2, 1 << 40)
    assert (n, n_pad, s) == (1 << 62, 1 << 62, 1 << 61)
    with pytest.raises(ValueError):
        oracle.dim0_layout([(big, 2)], 8)
    with pytest.raises(ValueError):
        oracle.dim0_layout([(1 << 40, 1 << 22), (1 << 40, 1 << 22)], 8)
