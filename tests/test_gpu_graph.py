"""The library's calls under HIP graph capture: a launch-bound loop (a
shard stepped in small buckets, "ZeRO and FSDP", A sharded Adam step) is
captured once and replayed.  The step's constants (bias corrections of step
t) are kernel arguments, so a graph replays the step it captured; each
replay here starts from the same state, restored eagerly between replays,
and must equal the eager result bit for bit -- weights, moments, the slot,
the overflow flag and the (fixed-order) sum of squares."""
import numpy as np
import pytest
import torch

import zero_sharded_mixed_flatten_amd as zs
from synth import BF16
from synth.workloads import GradDraw
from tests.gpu_util import dev16, devf, host_master, host_rows

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


def test_bucketed_step_replays_in_a_graph():
    n_dp, rank, S = 4, 1, 100_000
    buckets = [(0, 25_000), (25_000, 50_003), (50_003, 75_000), (75_000, S)]
    lay, _ = zs.zero_flatten_layout([S * n_dp], n_dp)
    draw = GradDraw(BF16, 1e-3)
    g = dev16(host_rows(252, 1, 0, n_dp, rank * S, S, draw), zs.ZERO_BF16)
    w0 = devf(host_master(252, rank * S, S))
    W, M, V = w0.clone(), torch.zeros(S, device="cuda"), torch.zeros(S, device="cuda")
    wf = torch.zeros(lay.n_pad, dtype=torch.bfloat16, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ss = torch.zeros(1, dtype=torch.float64, device="cuda")
    ws = torch.empty(zs.zero_sumsq_workspace_bytes(S) // 8 + 1, dtype=torch.float64,
                     device="cuda")
    hp = zs.AdamWHParams(step=1, grad_scale=1.0 / n_dp, **HP)

    def step(stream):
        flag.zero_()  # fill kernels, not memset nodes
        ss.zero_()
        for b0, b1 in buckets:
            zs.zero_shard_step(g.view(n_dp, S)[:, b0:], S, b1 - b0, W[b0:], M[b0:], V[b0:], wf,
                               lay, rank, hp, shard_off=b0, overflow=flag, sumsq=ss,
                               workspace=ws, stream=stream)

    def restore():
        W.copy_(w0)
        M.zero_()
        V.zero_()
        wf.zero_()

    # eager reference
    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [x.clone() for x in (W, M, V, wf, flag, ss)]

    # capture on a side stream, then replay three times from the restored state
    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for replay in range(3):
        restore()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("master", "m", "v", "weights", "flag", "sumsq"),
                                   (W, M, V, wf, flag, ss), ref):
            a, b = got.cpu(), want.cpu()
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), f"replay {replay}: {name} differs from the eager step"
    assert int(ref[4].item()) == 0 and float(ref[5].item()) > 0.0
