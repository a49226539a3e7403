"""The fused step for callers that cannot allocate, zero_shard_step_noalloc
(its sum of squares through the library's own device scratch), against
zero_shard_step with a caller workspace, through the C ABI.  Two calls in a
row, the second on a shorter range, each compared bit for bit with the
workspace call on a copy of the same inputs: master, m, v, the weight slot
(canaries outside it), the overflow flag and the sum of squares."""
import numpy as np
import pytest
import torch

import synth
import zero_sharded_mixed_flatten_amd as zs
from synth import BF16, F32, tag
from synth.synth_const import BUF_GRAD, BUF_MASTER, outlier_threshold

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
CANARY = -3.0


def _inputs(n_dp, S, rank, seed):
    dev = torch.device("cuda", 0)
    grads = torch.empty((n_dp, S), dtype=torch.bfloat16, device=dev)
    for k in range(n_dp):
        synth.fill_device(grads[k], BF16, seed, tag(BUF_GRAD, 170, 1, 0, k), rank * S, 1e-3,
                          outlier_threshold(0.01), 100.0)
    master = torch.empty(S, dtype=torch.float32, device=dev)
    synth.fill_device(master, F32, seed, tag(BUF_MASTER, 170), rank * S, 0.02)
    m = torch.empty(S, dtype=torch.float32, device=dev)
    synth.fill_device(m, F32, seed + 1, tag(BUF_MASTER, 171), rank * S, 1e-4)
    v = torch.empty(S, dtype=torch.float32, device=dev)
    synth.fill_device(v, F32, seed + 2, tag(BUF_MASTER, 172), rank * S, 1e-6)
    v.abs_()
    return grads, master, m, v


def _run(noalloc, grads, master, m, v, lay, rank, length, shard_off, t):
    S = lay.shard
    g, w, mm, vv = (x.clone() for x in (grads, master, m, v))
    wfull = torch.full((lay.n_pad,), CANARY, dtype=torch.bfloat16, device=w.device)
    flag = torch.zeros(1, dtype=torch.int32, device=w.device)
    ssq = torch.zeros(1, dtype=torch.float64, device=w.device)
    hp = zs.AdamWHParams(step=t, grad_scale=1.0 / lay.n_dp, **HP)
    args = (g[:, shard_off:], S, length, w[shard_off:], mm[shard_off:], vv[shard_off:], wfull,
            lay, rank, hp)
    if noalloc:
        zs.zero_shard_step_noalloc(*args, shard_off=shard_off, overflow=flag, sumsq=ssq)
    else:
        ws = torch.empty(zs.zero_sumsq_workspace_bytes(length) // 8 + 1, dtype=torch.float64,
                         device=w.device)
        zs.zero_shard_step(*args, shard_off=shard_off, overflow=flag, sumsq=ssq, workspace=ws)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in (w, mm, vv)] + [
        wfull.view(torch.int16).cpu().numpy(), int(flag.item()), float(ssq.item())]


def _same(a, b):
    """bitwise, NaN matching NaN"""
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype.kind == "f":
        na, nb = np.isnan(a), np.isnan(b)
        return np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32),
                                                         b[~nb].view(np.uint32))
    return np.array_equal(a, b)


@pytest.mark.parametrize("n_dp", [8, 3])
def test_noalloc_step_equals_the_workspace_step_on_two_calls(n_dp):
    """A long ragged range, then a shorter one at another shard offset (the
    scratch keeps the first call's partials; the second must not see them);
    the first call also meets an infinity in one gradient row."""
    S, rank = 4_194_304 + 1536, 1
    lay, _ = zs.zero_flatten_layout([S * n_dp], n_dp)
    grads, master, m, v = _inputs(n_dp, S, rank, seed=n_dp)
    grads[n_dp - 1, 777] = float("inf")
    for length, shard_off, t in ((S - 1003, 1001, 3), (300_007, 64, 4)):
        print(f"\n[no-alloc] n_dp={n_dp} len={length} off={shard_off} t={t}", flush=True)
        a = _run(True, grads, master, m, v, lay, rank, length, shard_off, t)
        b = _run(False, grads, master, m, v, lay, rank, length, shard_off, t)
        for x, y, what in zip(a, b, ("master", "m", "v", "weights", "overflow", "sumsq")):
            assert _same(x, y), what
        got_w = a[3]
        lo = rank * S + shard_off
        canary = np.array([CANARY], np.float32).view(np.uint32) >> 16
        assert np.all(got_w[:lo].view(np.uint16) == canary)
        assert np.all(got_w[lo + length:].view(np.uint16) == canary)
        assert a[4] == (1 if shard_off <= 777 < shard_off + length else 0)
        if a[4] == 0:
            assert np.isfinite(a[5]) and a[5] > 0


def test_noalloc_step_without_a_sum_and_at_the_length_limit():
    """Without a sum of squares no scratch is used and any length goes
    through; with one, a length past ZERO_NOALLOC_MAX_LEN is refused before
    anything runs."""
    n_dp, S, rank = 2, 65_536, 0
    lay, _ = zs.zero_flatten_layout([S * n_dp], n_dp)
    grads, master, m, v = _inputs(n_dp, S, rank, seed=5)
    w1, m1, v1, wf1, _, _ = _run(False, grads, master, m, v, lay, rank, S, 0, 2)
    w2, m2, v2 = master.clone(), m.clone(), v.clone()
    wf2 = torch.full((lay.n_pad,), CANARY, dtype=torch.bfloat16, device=w2.device)
    zs.zero_shard_step_noalloc(grads, S, S, w2, m2, v2, wf2, lay, rank,
                               zs.AdamWHParams(step=2, grad_scale=1.0 / n_dp, **HP))
    torch.cuda.synchronize()
    assert _same(w2.cpu().numpy(), w1) and _same(m2.cpu().numpy(), m1)
    assert _same(v2.cpu().numpy(), v1)
    assert np.array_equal(wf2.view(torch.int16).cpu().numpy(), wf1)
    big = zs.ZERO_NOALLOC_MAX_LEN + 4
    ssq = torch.zeros(1, dtype=torch.float64, device=w2.device)
    with pytest.raises(zs.ZeroValueError, match="ZERO_NOALLOC_MAX_LEN"):
        zs.zero_shard_step_noalloc(grads, big, big, w2, m2, v2, wf2, lay, rank,
                                   zs.AdamWHParams(step=3, grad_scale=0.5, **HP), sumsq=ssq)
    assert ssq.item() == 0.0
