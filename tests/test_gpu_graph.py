"""The library's calls under HIP graph capture: a launch-bound loop (a
shard stepped in small buckets, "ZeRO and FSDP", A sharded Adam step) is
captured once and replayed.  With the step's constants as kernel arguments
a graph replays the step it captured: each replay starts from the same
state, restored eagerly between replays, and must equal the eager result
bit for bit -- weights, moments, the slot, the overflow flag and the
(fixed-order) sum of squares.  With the constants in device memory (the _dc
entry points) one graph serves a run of steps, each replay checked against
the oracle's step, including a stage-2 step whose step number the host
holds back after an overflow."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_flatten_amd as zs
from synth import BF16, F16
from synth.workloads import GradDraw
from tests.gpu_util import dev16, devf, host16, host_master, host_rows, hostf

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


def test_one_graph_serves_every_step():
    """With the constants in device memory (zero_shard_step_dc) one captured
    graph serves a run of steps: before each replay the next step's
    constants (step t, a halving learning rate) and gradients are written
    into the buffers the graph reads, and every replay must equal the
    oracle's step t bit for bit."""
    n_dp, rank, S = 4, 1, 100_000
    buckets = [(0, 25_000), (25_000, 50_003), (50_003, 75_000), (75_000, S)]
    lay, _ = zs.zero_flatten_layout([S * n_dp], n_dp)
    draw = GradDraw(BF16, 1e-3)
    w = host_master(251, rank * S, S)
    m, v = np.zeros(S, np.float32), np.zeros(S, np.float32)
    wout = np.zeros(lay.n_pad, np.uint16)
    g = dev16(host_rows(251, 1, 0, n_dp, rank * S, S, draw), zs.ZERO_BF16)
    W, M, V = devf(w), devf(m), devf(v)
    wf = torch.zeros(lay.n_pad, dtype=torch.bfloat16, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ss = torch.zeros(1, dtype=torch.float64, device="cuda")
    ws = torch.empty(zs.zero_sumsq_workspace_bytes(S) // 8 + 1, dtype=torch.float64,
                     device="cuda")
    consts = zs.new_step_consts()

    def step(stream):
        flag.zero_()
        ss.zero_()
        for b0, b1 in buckets:
            zs.zero_shard_step_dc(g.view(n_dp, S)[:, b0:], S, b1 - b0, W[b0:], M[b0:], V[b0:], wf,
                                  lay, rank, consts, shard_off=b0, overflow=flag, sumsq=ss,
                                  workspace=ws, stream=stream)

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capture ran nothing: the state is still the initial one
    assert np.array_equal(hostf(W).view(np.uint32), w.view(np.uint32))
    for t in (1, 2, 3, 4):
        lr = 1e-4 / 2 ** (t - 1)
        hp = zs.AdamWHParams(step=t, grad_scale=1.0 / n_dp, **dict(HP, lr=lr))
        rows = host_rows(251, t, 0, n_dp, rank * S, S, draw)
        g.copy_(dev16(rows, zs.ZERO_BF16))
        consts.copy_(torch.from_numpy(zs.zero_step_consts_make(hp)))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_ovf, o_ss = np.zeros(1, np.uint32), np.zeros(1)
        slot = wout[rank * S:(rank + 1) * S].copy()
        oracle.step(rows, oracle.BF16, n_dp, S, S, w, m, v, slot, oracle.BF16, t,
                    grad_scale=1.0 / n_dp, overflow=o_ovf, sumsq=o_ss, **dict(HP, lr=lr))
        wout[rank * S:(rank + 1) * S] = slot
        for name, got, want in (("master", hostf(W), w), ("m", hostf(M), m), ("v", hostf(V), v)):
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"t={t}: {name}"
        assert np.array_equal(host16(wf), wout), f"t={t}: weights"
        assert int(flag.item()) == 0 and abs(ss.item() - o_ss[0]) <= 1e-10 * o_ss[0]


def test_stage2_graph_holds_the_step_back_after_an_overflow():
    """A stage-2 step -- two fp16 micro-batch reduces with the overflow
    flag, AdamW with the device constants gated on the flag and scaled by
    the device loss scale, the loss-scale update -- captured once and
    replayed for six iterations.  The host reads the flag after each replay
    and advances t only when the step was taken; an infinity injected in
    iteration 2 must skip that step (state untouched, scale backed off) and
    hold t back.  Every iteration equals the oracle's bit for bit."""
    n_dp, rank, S, micro = 4, 2, 50_000, 2
    lay, _ = zs.zero_flatten_layout([S * n_dp], n_dp)
    draw = GradDraw(F16, 1e-3, scale=65536.0)
    w = host_master(250, rank * S, S)
    m, v = np.zeros(S, np.float32), np.zeros(S, np.float32)
    wout = np.zeros(lay.n_pad, np.uint16)
    gb = [dev16(host_rows(250, 1, mb, n_dp, rank * S, S, draw), zs.ZERO_FP16)
          for mb in range(micro)]
    acc = torch.zeros(S, dtype=torch.float32, device="cuda")
    W, M, V = devf(w), devf(m), devf(v)
    wf = torch.zeros(lay.n_pad, dtype=torch.bfloat16, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    dls = zs.new_loss_scale(65536.0)
    consts = zs.new_step_consts()
    o_scale, o_good = np.array([65536.0], np.float32), np.zeros(1, np.int32)
    o_acc = np.zeros(S, np.float32)

    def step(stream):
        flag.zero_()
        for mb in range(micro):
            zs.zero_shard_reduce(gb[mb], n_dp, S, S, acc, accumulate=mb > 0, overflow=flag,
                                 stream=stream)
        zs.zero_shard_adamw_dc(acc, W, M, V, wf, lay, rank, consts, skip=flag, loss_scale=dls,
                               stream=stream)
        zs.zero_loss_scale_update(dls, flag, 2.0, 0.5, 3, stream=stream)

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    t, taken = 1, []
    for it in range(6):
        rows = [host_rows(250, it + 1, mb, n_dp, rank * S, S, draw) for mb in range(micro)]
        if it == 2:
            rows[1][3, 777] = 0x7C00                  # fp16 +inf in the last micro-batch
        for mb in range(micro):
            gb[mb].copy_(dev16(rows[mb], zs.ZERO_FP16))
        hp = zs.AdamWHParams(step=t, grad_scale=1.0 / (n_dp * micro), **HP)
        consts.copy_(torch.from_numpy(zs.zero_step_consts_make(hp)))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        skipped = int(flag.item()) != 0
        # the oracle, the same iteration
        o_flag = np.zeros(1, np.uint32)
        for mb in range(micro):
            oracle.reduce(rows[mb], oracle.FP16, n_dp, S, S, o_acc, int(mb > 0), overflow=o_flag)
        slot = wout[rank * S:(rank + 1) * S].copy()
        oracle.adamw_ex(o_acc, w, m, v, slot, oracle.BF16, S, t, grad_scale=1.0 / (n_dp * micro),
                        skip=o_flag, loss_scale=o_scale.copy(), **HP)
        wout[rank * S:(rank + 1) * S] = slot
        oracle.loss_scale_update(o_scale, o_good, int(o_flag[0]), 2.0, 0.5, 3)
        assert skipped == bool(o_flag[0]) == (it == 2), f"iteration {it}"
        for name, got, want in (("master", hostf(W), w), ("m", hostf(M), m), ("v", hostf(V), v)):
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"it={it}: {name}"
        assert np.array_equal(host16(wf), wout), f"it={it}: weights"
        assert zs.read_loss_scale(dls) == (float(o_scale[0]), int(o_good[0])), f"it={it}"
        taken.append(t)
        if not skipped:
            t += 1
    assert taken == [1, 2, 3, 3, 4, 5]


def test_stage2_graph_with_a_device_step_counter():
    """The stage-2 graph with the step counter on the device: it begins by
    selecting step t's constants from a table (steps 1..8) and ends by
    advancing t unless the overflow flag skipped the step, so the host
    writes neither constants nor t between replays -- only the next
    micro-batches' gradients.  An infinity in iteration 2 must skip that
    step and hold t at 3 for iteration 3; every iteration equals the
    oracle's bit for bit, and the device counter ends at 6."""
    n_dp, rank, S, micro = 4, 2, 50_000, 2
    lay, _ = zs.zero_flatten_layout([S * n_dp], n_dp)
    draw = GradDraw(F16, 1e-3, scale=65536.0)
    w = host_master(249, rank * S, S)
    m, v = np.zeros(S, np.float32), np.zeros(S, np.float32)
    wout = np.zeros(lay.n_pad, np.uint16)
    gb = [torch.zeros(n_dp * S, dtype=torch.float16, device="cuda") for _ in range(micro)]
    acc = torch.zeros(S, dtype=torch.float32, device="cuda")
    W, M, V = devf(w), devf(m), devf(v)
    wf = torch.zeros(lay.n_pad, dtype=torch.bfloat16, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    dls = zs.new_loss_scale(65536.0)
    gs = 1.0 / (n_dp * micro)
    table = zs.step_consts_table([zs.AdamWHParams(step=k, grad_scale=gs, **HP)
                                  for k in range(1, 9)])
    counter = zs.new_step_counter(1)
    consts = zs.new_step_consts()
    o_scale, o_good = np.array([65536.0], np.float32), np.zeros(1, np.int32)
    o_acc = np.zeros(S, np.float32)

    def step(stream):
        zs.zero_step_consts_select(consts, table, counter, stream=stream)
        flag.zero_()
        for mb in range(micro):
            zs.zero_shard_reduce(gb[mb], n_dp, S, S, acc, accumulate=mb > 0, overflow=flag,
                                 stream=stream)
        zs.zero_shard_adamw_dc(acc, W, M, V, wf, lay, rank, consts, skip=flag, loss_scale=dls,
                               stream=stream)
        zs.zero_loss_scale_update(dls, flag, 2.0, 0.5, 3, stream=stream)
        zs.zero_step_counter_advance(counter, skip=flag, stream=stream)

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert int(counter.item()) == 1  # capture ran nothing
    t = 1
    for it in range(6):
        rows = [host_rows(249, it + 1, mb, n_dp, rank * S, S, draw) for mb in range(micro)]
        if it == 2:
            rows[0][1, 4321] = 0x7C00                  # fp16 +inf in the first micro-batch
        for mb in range(micro):
            gb[mb].copy_(dev16(rows[mb], zs.ZERO_FP16).reshape(-1))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_flag = np.zeros(1, np.uint32)
        for mb in range(micro):
            oracle.reduce(rows[mb], oracle.FP16, n_dp, S, S, o_acc, int(mb > 0), overflow=o_flag)
        slot = wout[rank * S:(rank + 1) * S].copy()
        oracle.adamw_ex(o_acc, w, m, v, slot, oracle.BF16, S, t, grad_scale=gs, skip=o_flag,
                        loss_scale=o_scale.copy(), **HP)
        wout[rank * S:(rank + 1) * S] = slot
        oracle.loss_scale_update(o_scale, o_good, int(o_flag[0]), 2.0, 0.5, 3)
        if not o_flag[0]:
            t += 1
        assert bool(o_flag[0]) == (it == 2) and int(flag.item()) == int(o_flag[0])
        assert int(counter.item()) == t, f"iteration {it}"
        for name, got, want in (("master", hostf(W), w), ("m", hostf(M), m), ("v", hostf(V), v)):
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"it={it}: {name}"
        assert np.array_equal(host16(wf), wout), f"it={it}: weights"
        assert zs.read_loss_scale(dls) == (float(o_scale[0]), int(o_good[0])), f"it={it}"
    assert t == 6


def test_step_beyond_the_table_selects_nan_constants():
    table = zs.step_consts_table([zs.AdamWHParams(step=k) for k in (1, 2)])
    consts = zs.new_step_consts()
    for k, want in ((1, 0), (2, 1), (0, None), (3, None), (-5, None)):
        zs.zero_step_consts_select(consts, table, zs.new_step_counter(k))
        got = consts.cpu().numpy()
        if want is None:
            assert np.all(np.isnan(got[:40].view(np.float32))) and np.isnan(got[40:].view(np.float64)[0])
        else:
            assert np.array_equal(got, table[want].cpu().numpy())


def test_steps_past_the_table_are_held():
    """A counter past its table selects NaN constants; every device-constant
    entry point then holds the step: master, m, v, the weight slot, the
    8-bit codes and scales keep every bit, the overflow flag goes up, the
    sum of squares gets nothing, and the counter, advanced with that flag
    as skip, stays where it is.  A shard with a ragged tail, so that the
    element kernels hold too."""
    n_dp, rank, S = 4, 1, 50_003
    lay, _ = zs.zero_flatten_layout([S * n_dp], n_dp)
    table = zs.step_consts_table([zs.AdamWHParams(step=k, grad_scale=1.0 / n_dp, **HP)
                                  for k in (1, 2)])
    consts = zs.new_step_consts()
    t = zs.new_step_counter(3)
    zs.zero_step_consts_select(consts, table, t)
    rows = dev16(host_rows(201, 1, 0, n_dp, 0, S, GradDraw(BF16, 1e-3)), 0).view(n_dp, S)
    W0 = devf(host_master(202, 0, S))
    M0 = devf(host_master(203, 0, S, sigma=1e-4))
    V0 = devf(np.abs(host_master(204, 0, S, sigma=1e-6)))
    W, M, V = W0.clone(), M0.clone(), V0.clone()
    wf = torch.full((lay.n_pad,), -2.0, dtype=torch.bfloat16, device="cuda")
    wf0 = wf.clone()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ss = torch.zeros(1, dtype=torch.float64, device="cuda")
    zs.zero_shard_step_dc(rows, S, S, W, M, V, wf, lay, rank, consts, overflow=flag, sumsq=ss)
    acc = devf(host_master(205, 0, S, sigma=1e-3))
    zs.zero_shard_adamw_dc(acc, W, M, V, wf, lay, rank, consts)
    zs.zero_step_counter_advance(t, skip=flag)
    torch.cuda.synchronize()
    for got, want in ((W, W0), (M, M0), (V, V0), (wf, wf0)):
        assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else
                           got.view(torch.int32),
                           want.view(torch.int16) if want.dtype == torch.bfloat16 else
                           want.view(torch.int32))
    assert int(flag.item()) == 1 and ss.item() == 0.0 and int(t.item()) == 3
    # the 8-bit step
    B = zs.ZERO_Q8_BLOCK
    Sq = 40 * B + 77
    layq, _ = zs.zero_flatten_layout([Sq * n_dp], n_dp, B)
    Sq = layq.shard
    x = devf(host_master(206, 0, n_dp * Sq, sigma=1e-3))
    gq = torch.empty(n_dp * Sq, dtype=torch.int8, device="cuda")
    gs = torch.empty(zs.q8_blocks(n_dp * Sq), device="cuda")
    zs.zero_q8_quantize(x, gq, gs)
    Wq0 = devf(host_master(207, 0, Sq))
    Wq, Mq, Vq = Wq0.clone(), torch.zeros(Sq, device="cuda"), torch.zeros(Sq, device="cuda")
    wq = torch.full((layq.n_pad,), 5, dtype=torch.int8, device="cuda")
    wsc = torch.full((layq.n_pad // B,), 0.25, device="cuda")
    flag.zero_()
    zs.zero_shard_step_q8_dc(gq, gs, Sq, Sq // B, Sq, Wq, Mq, Vq, wq, wsc, layq, rank, consts,
                             overflow=flag)
    torch.cuda.synchronize()
    assert torch.equal(Wq.view(torch.int32), Wq0.view(torch.int32))
    assert not Mq.any() and not Vq.any()
    assert bool((wq == 5).all()) and bool((wsc == 0.25).all()) and int(flag.item()) == 1


def test_counter_advances_unless_skipped():
    t = zs.new_step_counter(41)
    zs.zero_step_counter_advance(t)                                    # no flag: advance
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_step_counter_advance(t, skip=flag)                         # flag clear: advance
    flag.fill_(1)
    zs.zero_step_counter_advance(t, skip=flag)                         # flag set: hold
    assert int(t.item()) == 43


def test_device_constants_keep_grad_scale_in_double():
    """With a dynamic loss scale, s = fl(grad_scale / scale) is formed from
    the double grad_scale: for grad_scale = 1/12 (not an fp32 value) the
    device-constant AdamW must equal the hp-taking one bit for bit, which it
    would not if it divided the fp32-rounded scale instead."""
    S, gs, scale = 40_000, 1.0 / 12, 65535.0
    # the two readings of s differ for these values (a power-of-two scale
    # would not tell them apart: dividing by it commutes with rounding)
    assert np.float32(gs / scale) != np.float32(float(np.float32(gs)) / scale)
    lay, _ = zs.zero_flatten_layout([S], 1)
    acc = devf(host_master(248, 0, S, sigma=1e-3 * scale))
    outs = []
    for dc in (False, True):
        W, M, V = devf(host_master(247, 0, S)), torch.zeros(S, device="cuda"), torch.zeros(S, device="cuda")
        wf = torch.zeros(S, dtype=torch.bfloat16, device="cuda")
        ls = zs.new_loss_scale(scale)
        for t in (1, 2):
            hp = zs.AdamWHParams(step=t, grad_scale=gs, **HP)
            if dc:
                consts = zs.new_step_consts()
                consts.copy_(torch.from_numpy(zs.zero_step_consts_make(hp)))
                zs.zero_shard_adamw_dc(acc, W, M, V, wf, lay, 0, consts, loss_scale=ls)
            else:
                zs.zero_shard_adamw_ex(acc, W, M, V, wf, lay, 0, hp, loss_scale=ls)
        torch.cuda.synchronize()
        outs.append([hostf(W), hostf(M), hostf(V), host16(wf)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    # and the oracle agrees
    w, m, v = host_master(247, 0, S), np.zeros(S, np.float32), np.zeros(S, np.float32)
    wo = np.zeros(S, np.uint16)
    for t in (1, 2):
        oracle.adamw_ex(hostf(acc), w, m, v, wo, oracle.BF16, S, t, grad_scale=gs,
                        loss_scale=np.array([scale], np.float32), **HP)
    assert np.array_equal(outs[0][0].view(np.uint32), w.view(np.uint32))
