"""GPU parity of the functional sharded Adam step ("ZeRO and FSDP", "A
sharded Adam step": n_dp simulated ranks, each rank's full local gradient,
np.array_split shards of fp32 master and moments, reduce-scatter of the
average, Adam with bias correction from t = 1, all-gather; inputs not
modified) against the oracle, bit for bit, through the C ABI's kernels."""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_flatten_amd as zs
from synth import BF16, F32, tag
from synth.synth_const import BUF_GRAD, BUF_MASTER

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, b1=0.9, b2=0.999, eps=1e-8)


@pytest.mark.parametrize("n_dp", [1, 3, 4, 8])
@pytest.mark.parametrize("kind", [F32, BF16])
def test_functional_step_matches_oracle(n_dp, kind):
    n = 10_007
    pieces = np.array_split(np.arange(n), n_dp)
    starts = [int(p[0]) if p.size else 0 for p in pieces]
    w0 = synth.fill_host(F32, 0, tag(BUF_MASTER, 140), 0, n, 0.02)
    ws = [torch.from_numpy(w0[p].copy()).cuda() for p in pieces]
    ms = [torch.zeros(p.size, device="cuda") for p in pieces]
    vs = [torch.zeros(p.size, device="cuda") for p in pieces]
    o_w = [w0[p].copy() for p in pieces]
    o_m = [np.zeros(p.size, np.float32) for p in pieces]
    o_v = [np.zeros(p.size, np.float32) for p in pieces]
    gdt = oracle.FP32 if kind == F32 else oracle.BF16
    for t in (1, 2, 3):
        g_host = np.stack([synth.fill_host(kind, 0, tag(BUF_GRAD, 140, t, 0, k), 0, n, 1e-3)
                           for k in range(n_dp)])
        if kind == F32:
            grads = [torch.from_numpy(g_host[k].copy()).cuda() for k in range(n_dp)]
        else:
            grads = [torch.from_numpy(g_host[k].view(np.int16).copy()).cuda().view(torch.bfloat16)
                     for k in range(n_dp)]
        before = [x.clone() for x in grads + ws + ms + vs]
        full_w, ws2, ms2, vs2 = zs.zero_adam_step(grads, ws, ms, vs, t, **HP)
        torch.cuda.synchronize()
        for a, b in zip(before, grads + ws + ms + vs):  # inputs untouched
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
        for r, p in enumerate(pieces):
            if p.size == 0:
                continue
            acc = np.zeros(p.size, np.float32)
            oracle.reduce(g_host.reshape(-1)[starts[r]:], gdt, n_dp, n, p.size, acc, 0)
            wout = np.zeros(p.size, np.uint16)
            oracle.adamw(acc, o_w[r], o_m[r], o_v[r], wout, oracle.BF16, p.size, t, lr=HP["lr"],
                         beta1=HP["b1"], beta2=HP["b2"], eps=HP["eps"], weight_decay=0.0,
                         grad_scale=1.0 / n_dp)
        for got, ref in ((ws2, o_w), (ms2, o_m), (vs2, o_v)):
            for x, y in zip(got, ref):
                assert np.array_equal(x.cpu().numpy().view(np.uint32), y.view(np.uint32))
        whole = np.concatenate(o_w)
        assert len(full_w) == n_dp
        for f in full_w:
            assert np.array_equal(f.cpu().numpy().view(np.uint32), whole.view(np.uint32))
        ws, ms, vs = ws2, ms2, vs2


def test_functional_step_on_a_side_stream():
    """Given a stream, the functional step runs (and allocates) there: its
    results equal the same step on the current stream bit for bit, with
    the current stream allocating and overwriting memory meanwhile."""
    n_dp, n = 4, 1_000_003
    pieces = np.array_split(np.arange(n), n_dp)
    w0 = synth.fill_host(F32, 0, tag(BUF_MASTER, 141), 0, n, 0.02)
    g_host = np.stack([synth.fill_host(F32, 0, tag(BUF_GRAD, 141, 1, 0, k), 0, n, 1e-3)
                       for k in range(n_dp)])
    grads = [torch.from_numpy(g_host[k].copy()).cuda() for k in range(n_dp)]

    def state():
        return ([torch.from_numpy(w0[p].copy()).cuda() for p in pieces],
                [torch.zeros(p.size, device="cuda") for p in pieces],
                [torch.zeros(p.size, device="cuda") for p in pieces])

    ref = zs.zero_adam_step(grads, *state(), 1, **HP)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    st = state()
    side.wait_stream(torch.cuda.current_stream())
    got = zs.zero_adam_step(grads, *st, 1, stream=side, **HP)
    junk = [torch.empty(n, device="cuda").fill_(float("nan")) for _ in range(8)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del junk
    for a_list, b_list in zip(ref, got):
        for a, b in zip(a_list, b_list):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_functional_step_more_ranks_than_elements():
    """n < n_dp: array_split leaves some ranks an empty piece."""
    n, n_dp = 5, 8
    grads = [torch.full((n,), float(k + 1), device="cuda") for k in range(n_dp)]
    pieces = np.array_split(np.arange(n), n_dp)
    ws = [torch.ones(p.size, device="cuda") for p in pieces]
    ms = [torch.zeros(p.size, device="cuda") for p in pieces]
    vs = [torch.zeros(p.size, device="cuda") for p in pieces]
    full_w, ws2, _, _ = zs.zero_adam_step(grads, ws, ms, vs, 1, **HP)
    torch.cuda.synchronize()
    # step 1 of Adam moves every weight by lr against the (positive) gradient, up to eps
    for f in full_w:
        assert torch.allclose(f, torch.full((n,), 1.0 - HP["lr"], device="cuda"), rtol=0, atol=1e-6)
    assert [x.numel() for x in ws2] == [p.size for p in pieces]


def test_functional_step_rejects_mismatched_shards():
    grads = [torch.zeros(10, device="cuda") for _ in range(2)]
    ws = [torch.zeros(5, device="cuda"), torch.zeros(4, device="cuda")]
    with pytest.raises(ValueError):
        zs.zero_adam_step(grads, ws, ws, ws, 1)
