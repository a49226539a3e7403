"""Calls on two HIP streams at once: the two halves of a shard stepped as
buckets on separate streams, each with its own workspace, both adding into
one sum of squares and one overflow flag (the header allows calls on other
streams to add to the same scalars; only a shared workspace must not be
used concurrently).  Every element must equal the oracle's bit for bit, the
untouched weight buffer its canaries, the flag the OR of both halves and the
sum the oracle's within its bound (the halves' partials are added in another
order than one whole-range call).  The arithmetic is "ZeRO and FSDP", A
sharded Adam step."""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_flatten_amd as zs
from synth import BF16
from synth.synth_const import BUF_GRAD
from synth.workloads import GradDraw
from tests.gpu_util import check_16, check_f32, dev16, devf, host16, host_master, host_rows, hostf

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
CANARY = 0x5A5A


def test_two_streams_add_into_one_sum_and_flag():
    n_dp, rank, S = 4, 2, 600_000
    halves = [(0, 300_001), (300_001, S)]      # the second starts off alignment
    lay, _ = zs.zero_flatten_layout([S * n_dp], n_dp)
    draw = GradDraw(BF16, 1e-3, outlier_p=0.01, outlier_mul=100.0)
    lo = rank * S
    w = host_master(253, lo, S)
    m, v = np.zeros(S, np.float32), np.zeros(S, np.float32)
    wout = np.full(lay.n_pad, CANARY, np.uint16)
    dw, dm, dv = devf(w), devf(m), devf(v)
    dwf = dev16(wout, zs.ZERO_BF16)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ss = torch.zeros(1, dtype=torch.float64, device="cuda")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [torch.empty(zs.zero_sumsq_workspace_bytes(b1 - b0) // 8, dtype=torch.float64,
                       device="cuda") for b0, b1 in halves]
    for t in (1, 2, 3):
        rows = host_rows(253, t, 0, n_dp, lo, S, draw)
        if t == 3:
            rows[3, 450_000] = 0x7F80            # +inf in the second half only
        g = dev16(rows, zs.ZERO_BF16)
        flag.zero_()
        ss.zero_()
        hp = zs.AdamWHParams(step=t, grad_scale=1.0 / n_dp, **HP)
        for (b0, b1), st, ws in zip(halves, streams, wss):
            st.wait_stream(torch.cuda.current_stream())
            zs.zero_shard_step(g[:, b0:], S, b1 - b0, dw[b0:], dm[b0:], dv[b0:], dwf, lay, rank,
                               hp, shard_off=b0, overflow=flag, sumsq=ss, workspace=ws, stream=st)
        for st in streams:
            torch.cuda.current_stream().wait_stream(st)
        o_ovf, o_ss = np.zeros(1, np.uint32), np.zeros(1)
        slot = wout[lo:lo + S].copy()
        oracle.step(np.ascontiguousarray(rows), oracle.BF16, n_dp, S, S, w, m, v, slot,
                    oracle.BF16, t, grad_scale=1.0 / n_dp, overflow=o_ovf, sumsq=o_ss, **HP)
        wout[lo:lo + S] = slot
        torch.cuda.synchronize()
        # (at t = 3 the inf makes that element's state NaN on both sides:
        # NaN positions are compared by class)
        diff = check_f32(hostf(dw), w, f"master t={t}") + check_f32(hostf(dm), m, f"m t={t}")
        diff += check_f32(hostf(dv), v, f"v t={t}")
        got = host16(dwf)
        diff += check_16(got[lo:lo + S], wout[lo:lo + S], zs.ZERO_BF16, f"weights t={t}")
        assert diff == 0
        assert np.array_equal(got[:lo], wout[:lo]) and np.array_equal(got[lo + S:], wout[lo + S:])
        assert int(flag.item()) == int(o_ovf[0]) == (1 if t == 3 else 0)
        if t < 3:
            assert abs(ss.item() - o_ss[0]) <= 1e-10 * o_ss[0]
        else:
            assert not np.isfinite(ss.item()) and not np.isfinite(o_ss[0])


def test_binding_workspace_lives_on_the_calls_stream():
    """A sum of squares asked for on a side stream without a workspace: the
    binding's temporary workspace is freed when the call returns, so it
    must belong to the call's stream.  Right after the call the current
    stream takes blocks of the same size and fills them with NaN while the
    side stream's step is still running; the step's sum must still equal
    the reduce's sum of the same rows over 64 (s = 1/8 is a power of two,
    and the order of both sums is fixed by the length alone)."""
    n_dp, S = 8, 1 << 26
    lay, _ = zs.zero_flatten_layout([S * n_dp], n_dp)
    rows = torch.empty((n_dp, S), dtype=torch.bfloat16, device="cuda")
    for k in range(n_dp):
        synth.fill_device(rows[k], BF16, 0, synth.tag(BUF_GRAD, 254, 1, 0, k), 0, 1e-3)
    acc = torch.empty(S, dtype=torch.float32, device="cuda")
    ref = torch.zeros(1, dtype=torch.float64, device="cuda")
    zs.zero_shard_reduce(rows, n_dp, S, S, acc, sumsq=ref)
    del acc
    W = torch.zeros(S, device="cuda")
    M, V = torch.zeros(S, device="cuda"), torch.zeros(S, device="cuda")
    wf = torch.zeros(lay.n_pad, dtype=torch.bfloat16, device="cuda")
    ss = torch.zeros(1, dtype=torch.float64, device="cuda")
    ws_elems = (zs.zero_sumsq_workspace_bytes(S) + 7) // 8
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        ss.zero_()
        torch.cuda.synchronize()
        zs.zero_shard_step(rows, S, S, W, M, V, wf, lay, 0,
                           zs.AdamWHParams(step=1, grad_scale=1.0 / n_dp, **HP), sumsq=ss,
                           stream=side)
        junk = [torch.empty(ws_elems, dtype=torch.float64, device="cuda").fill_(float("nan"))
                for _ in range(4)]
        torch.cuda.synchronize()
        del junk
        assert ss.item() == ref.item() / 64.0
