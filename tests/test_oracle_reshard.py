"""Pins of the oracle's re-sharding (CPU only): converting a sharded
checkpoint to another GPU count or consolidating it ("ZeRO Optimizer, in
depth", "Checkpoints: sharded on the way in, consolidated on the way out",
and "Failure modes seen in practice": resume fails after changing the GPU
count unless the checkpoint is converted)."""
import numpy as np
import pytest

import oracle


def _shards(flat, n_dp, align=1):
    _, n, n_pad, s = oracle.flatten_layout([flat.size], n_dp, align)
    padded = np.zeros(n_pad, flat.dtype)
    padded[:n] = flat
    return [padded[r * s:(r + 1) * s].copy() for r in range(n_dp)]


@pytest.mark.parametrize("n,a,b", [(10_000, 4, 3), (12_345, 8, 64), (777, 1, 8), (1000, 7, 1),
                                   (5, 8, 2), (0, 4, 2)])
@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_reshard_equals_slicing_of_the_flat_vector(n, a, b, dtype):
    rng = np.random.default_rng(n + a * 100 + b)
    flat = rng.integers(1, 60000, size=n).astype(dtype)
    old = _shards(flat, a)
    new_ref = _shards(flat, b)
    for r in range(b):
        assert np.array_equal(oracle.reshard(old, n, b, r), new_ref[r])


@pytest.mark.parametrize("a,b", [(8, 3), (3, 64), (64, 8)])
def test_round_trip_is_identity(a, b):
    n = 100_003
    flat = np.random.default_rng(a * b).standard_normal(n).astype(np.float32)
    old = _shards(flat, a)
    mid = [oracle.reshard(old, n, b, r) for r in range(b)]
    back = [oracle.reshard(mid, n, a, r) for r in range(a)]
    for x, y in zip(old, back):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_consolidation_recovers_every_tensor():
    """n_dp' = 1 consolidates: the flat vector, and through the offsets
    every parameter tensor, as zero_to_fp32 would write them."""
    numels = [300, 17, 4096, 1]
    offs, n, _, _ = oracle.flatten_layout(numels, 8)
    tensors = [np.random.default_rng(i).standard_normal(k).astype(np.float32)
               for i, k in enumerate(numels)]
    flat = np.concatenate(tensors)
    full = oracle.reshard(_shards(flat, 8), n, 1, 0)
    for t, o, k in zip(tensors, offs, numels):
        assert np.array_equal(full[o:o + k], t)


def _flat_of(pieces, n):
    """numpy: the flat vector a piece list describes (zeros where none)."""
    flat = np.zeros(n, pieces[0][0].dtype)
    for a, o in pieces:
        lo, hi = max(o, 0), min(o + a.size, n)
        if hi > lo:
            flat[lo:hi] = a[lo - o:hi - o]
    return flat


def _random_pieces(rng, n, dtype, gaps=True):
    cuts = np.sort(rng.choice(np.arange(1, n), size=min(n - 1, 12), replace=False))
    bounds = [0] + list(cuts) + [n]
    pieces = []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        if gaps and rng.random() < 0.25:
            continue  # a hole: gathers as zeros
        pieces.append((rng.integers(1, 60000, size=hi - lo).astype(dtype), int(lo)))
    rng.shuffle(pieces)  # piece order does not matter
    return pieces


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_gather_is_slicing_of_the_flat_vector(seed, dtype):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(50, 3000))
    pieces = _random_pieces(rng, n, dtype)
    if not pieces:
        pieces = [(np.ones(3, dtype), 0)]
    flat = _flat_of(pieces, n)
    for begin, count in [(0, n), (7, n - 20), (n - 5, 40), (n + 3, 9), (0, 0)]:
        want = np.zeros(count, dtype)
        lo, hi = min(max(begin, 0), n), min(begin + count, n)
        if hi > lo:
            want[lo - begin:hi - begin] = flat[lo:hi]
        assert np.array_equal(oracle.flat_gather(pieces, n, begin, count), want)


def test_locate_brute_force():
    pieces = [(np.zeros(5, np.float32), 10), (np.zeros(3, np.float32), 0), (np.zeros(2, np.float32), 20)]
    meta = [(o, a.size) for a, o in pieces]
    want = {0: (1, 0), 2: (1, 2), 3: (-1, None), 10: (0, 0), 14: (0, 4), 15: (-1, None),
            21: (2, 1), 22: (-1, None)}
    for i in range(25):
        held = [(k, i - o) for k, (o, ln) in enumerate(meta) if o <= i < o + ln and i < 22]
        assert oracle.flat_locate(meta, 22, i) == (held[0] if held else (-1, None))
    for i, kv in want.items():
        assert oracle.flat_locate(meta, 22, i) == kv
    assert oracle.flat_locate(meta, 21, 21) == (-1, None)  # beyond n


@pytest.mark.parametrize("a,b", [(8, 3), (4, 64), (1, 8)])
def test_gather_of_equal_shards_equals_reshard(a, b):
    """The two independently written forms agree."""
    n = 50_001
    flat = np.random.default_rng(a + b).standard_normal(n).astype(np.float32)
    old = _shards(flat, a)
    s_old = old[0].size
    pieces = [(x, r * s_old) for r, x in enumerate(old)]
    _, _, _, s_new = oracle.flatten_layout([n], b, 1)
    for r in range(b):
        assert np.array_equal(oracle.flat_gather(pieces, n, r * s_new, s_new),
                              oracle.reshard(old, n, b, r))


@pytest.mark.parametrize("seed", range(4))
def test_scatter_after_gather_is_identity(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(100, 2000))
    pieces = _random_pieces(rng, n, np.uint16, gaps=False)
    flat = _flat_of(pieces, n)
    begin = int(rng.integers(0, n // 2))
    count = int(rng.integers(1, n - begin))
    rng_vals = rng.integers(1, 60000, size=count).astype(np.uint16)
    dests = [(a.copy(), o) for a, o in pieces]
    oracle.flat_scatter(rng_vals, begin, dests)
    want = flat.copy()
    want[begin:begin + count] = rng_vals
    assert np.array_equal(_flat_of(dests, n), want)  # written inside the range, kept outside
    assert np.array_equal(oracle.flat_gather(dests, n, begin, count), rng_vals)


def test_flatten_then_unflatten_per_tensor():
    """Flattening gathers a rank's shard from the parameter tensors (pieces at
    their offsets); consolidation scatters every shard back into per-tensor
    buffers, which then equal the parameters."""
    numels = [1000, 3, 77, 4096, 1, 513]
    n_dp = 8
    offs, n, _, s = oracle.flatten_layout(numels, n_dp, 4)
    rng = np.random.default_rng(9)
    tensors = [rng.standard_normal(k).astype(np.float32) for k in numels]
    pieces = list(zip(tensors, offs))
    shards = [oracle.flat_gather(pieces, n, r * s, s) for r in range(n_dp)]
    assert np.array_equal(np.concatenate(shards)[:n], np.concatenate(tensors))
    assert not np.any(np.concatenate(shards)[n:])
    outs = [(np.zeros(k, np.float32), o) for k, o in zip(numels, offs)]
    for r, sh in enumerate(shards):
        oracle.flat_scatter(sh, r * s, outs)
    for (o, _), t in zip(outs, tensors):
        assert np.array_equal(o, t)
