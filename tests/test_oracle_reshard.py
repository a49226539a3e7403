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
