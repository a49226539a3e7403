"""The Python binding refuses, before any launch, tensors that do not fit the
sizes passed beside them: the C ABI takes plain pointers and cannot see a
tensor's extent, so a short, strided, expanded or host tensor must be
caught here.  Every call below raises and leaves its canaries untouched."""
import pytest
import torch

import zero_sharded_mixed_flatten_amd as zs

pytestmark = pytest.mark.gpu

HP = zs.AdamWHParams(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1,
                     grad_scale=0.25, step=1)


def _step_args(S=1024, n_dp=4, rank=1):
    lay, _ = zs.zero_flatten_layout([S * n_dp], n_dp)
    g = torch.zeros(n_dp * S, dtype=torch.bfloat16, device="cuda")
    W = torch.full((S,), 3.0, device="cuda")
    M = torch.zeros(S, device="cuda")
    V = torch.zeros(S, device="cuda")
    wf = torch.full((lay.n_pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    return lay, g, W, M, V, wf


def _untouched(W, wf):
    torch.cuda.synchronize()
    assert bool((W == 3.0).all()) and bool((wf == 7.0).all())


def test_step_refuses_short_and_strided_tensors():
    lay, g, W, M, V, wf = _step_args()
    S = lay.shard
    with pytest.raises(ValueError, match="master"):
        zs.zero_shard_step(g, S, S, W[:S - 1], M, V, wf, lay, 1, HP)
    with pytest.raises(ValueError, match="grads"):
        zs.zero_shard_step(g[:3 * S + S - 1], S, S, W, M, V, wf, lay, 1, HP)
    with pytest.raises(ValueError, match="weight_full"):
        zs.zero_shard_step(g, S, S, W, M, V, wf[:2 * S - 1], lay, 1, HP)
    big = torch.zeros(2 * S, device="cuda")
    with pytest.raises(TypeError, match="contiguous"):
        zs.zero_shard_step(g, S, S, W, big[::2], V, wf, lay, 1, HP)
    with pytest.raises(TypeError, match="contiguous"):
        zs.zero_shard_step(g, S, S, W, M, torch.zeros(1, device="cuda").expand(S), wf, lay, 1, HP)
    with pytest.raises(TypeError, match="GPU tensor"):
        zs.zero_shard_step(g, S, S, W, M, V.cpu(), wf, lay, 1, HP)
    # rows as a 2-D view of row stride ld: the stride must be ld and the
    # view must hold n_dp rows of len elements
    g2 = g.view(4, S)
    with pytest.raises(TypeError, match="row stride"):
        zs.zero_shard_step(g2[:, ::2], S, S // 2, W, M, V, wf, lay, 1, HP)
    with pytest.raises(ValueError, match="grads"):
        zs.zero_shard_step(g2[:, 8:], S, S, W, M, V, wf, lay, 1, HP)
    with pytest.raises(ValueError, match="overflow"):
        zs.zero_shard_step(g, S, S, W, M, V, wf, lay, 1, HP,
                           overflow=torch.zeros(0, dtype=torch.int32, device="cuda"))
    _untouched(W, wf)
    # the same call with fitting tensors runs
    zs.zero_shard_step(g, S, S, W, M, V, wf, lay, 1, HP)
    torch.cuda.synchronize()


def test_reduce_and_adamw_refuse_short_tensors():
    lay, g, W, M, V, wf = _step_args()
    S = lay.shard
    acc = torch.full((S,), 5.0, device="cuda")
    with pytest.raises(ValueError, match="acc"):
        zs.zero_shard_reduce(g, 4, S, S, acc[:S - 4])
    with pytest.raises(ValueError, match="grads"):
        zs.zero_shard_reduce(g[:S], 4, S, S, acc)
    with pytest.raises(ValueError, match="v"):
        zs.zero_shard_adamw(acc, W, M, V[:S - 1], wf, lay, 1, HP)
    with pytest.raises(ValueError, match="weight_full"):
        zs.zero_shard_adamw(acc, W, M, V, wf[:S], lay, 1, HP)
    with pytest.raises(ValueError, match="loss_scale"):
        zs.zero_shard_adamw_ex(acc, W, M, V, wf, lay, 1, HP,
                               loss_scale=torch.zeros(1, dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError, match="loss_scale"):
        zs.zero_loss_scale_update(torch.zeros(1, dtype=torch.int32, device="cuda"),
                                  torch.zeros(1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert bool((acc == 5.0).all())
    _untouched(W, wf)


def test_codec_refuses_short_tensors():
    n = 1000
    x = torch.ones(n, device="cuda")
    q = torch.full((n,), 9, dtype=torch.int8, device="cuda")
    s = torch.full((zs.q8_blocks(n),), 2.0, device="cuda")
    y = torch.full((n,), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="q"):
        zs.zero_q8_quantize(x, q[:n - 1], s)
    with pytest.raises(ValueError, match="scales"):
        zs.zero_q8_quantize(x, q, s[:zs.q8_blocks(n) - 1])
    with pytest.raises(ValueError, match="y"):
        zs.zero_q8_dequantize(q, s, y[:n - 1])
    with pytest.raises(ValueError, match="scales"):
        zs.zero_q8_dequantize(q, s[:1], y)
    torch.cuda.synchronize()
    assert bool((q == 9).all()) and bool((s == 2.0).all()) and bool((y == 7.0).all())


def test_q8_step_refuses_short_tensors():
    B = zs.ZERO_Q8_BLOCK
    n_dp, S = 2, 4 * B
    lay, _ = zs.zero_flatten_layout([S * n_dp], n_dp, B)
    gq = torch.zeros(n_dp * S, dtype=torch.int8, device="cuda")
    gs = torch.ones(n_dp * (S // B), device="cuda")
    W = torch.full((S,), 3.0, device="cuda")
    M = torch.zeros(S, device="cuda")
    V = torch.zeros(S, device="cuda")
    wq = torch.full((lay.n_pad,), 7, dtype=torch.int8, device="cuda")
    ws = torch.full((lay.n_pad // B,), 7.0, device="cuda")
    args = (S, S // B, S, W, M, V)
    with pytest.raises(ValueError, match="gq"):
        zs.zero_shard_step_q8(gq[:S + S - 1], gs, *args, wq, ws, lay, 1, HP)
    with pytest.raises(ValueError, match="gscales"):
        zs.zero_shard_step_q8(gq, gs[:S // B + 1], *args, wq, ws, lay, 1, HP)
    with pytest.raises(ValueError, match="wq_full"):
        zs.zero_shard_step_q8(gq, gs, *args, wq[:2 * S - 1], ws, lay, 1, HP)
    with pytest.raises(ValueError, match="wscales_full"):
        zs.zero_shard_step_q8(gq, gs, *args, wq, ws[:2 * S // B - 1], lay, 1, HP)
    torch.cuda.synchronize()
    assert bool((W == 3.0).all()) and bool((wq == 7).all()) and bool((ws == 7.0).all())
    zs.zero_shard_step_q8(gq, gs, *args, wq, ws, lay, 1, HP)
    torch.cuda.synchronize()
