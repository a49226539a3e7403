"""GPU parity of the step controls (through the C ABI): the fp16 stage-2
step with a dynamic loss scale and global-norm clipping, for every rank of
a small data-parallel group emulated on one GPU, against the oracle.

The whole-model sum of squares is the sum of the ranks' partials.  For the
bit-exact comparison both sides take the oracle's float64 sum (the GPU's
own partials are order dependent, checked within 1e-10); a second test runs
the all-GPU pipeline end to end against the stated bar."""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_flatten_amd as zs
from synth import F16
from synth.workloads import GradDraw
from tests.gpu_util import check_16, check_f32, dev16, devf, host16, host_master, host_rows, hostf

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
DRAW = GradDraw(F16, 1e-3, scale=65536.0)


def _group(n_dp, numel, cfg):
    lay, _ = zs.zero_flatten_layout([numel], n_dp, 8)
    ranks = []
    for r in range(n_dp):
        s = lay.shard
        w = host_master(cfg, r * s, s, pad_from=numel)
        ranks.append(dict(w=w, m=np.zeros(s, np.float32), v=np.zeros(s, np.float32),
                          dw=devf(w), dm=devf(np.zeros(s, np.float32)),
                          dv=devf(np.zeros(s, np.float32)), dacc=devf(np.zeros(s, np.float32)),
                          acc=np.zeros(s, np.float32)))
    return lay, ranks


def _rows(cfg, t, mb, n_dp, lo, s, numel, loss_scale, inject):
    rows = host_rows(cfg, t, mb, n_dp, lo, s, DRAW, pad_from=numel)
    if loss_scale != 65536.0:  # the draw is at scale 65536; rescale exactly (powers of two)
        f = oracle.f16_to_f32(rows) * np.float32(loss_scale / 65536.0)
        rows = oracle.f32_to_f16(f)
    if inject is not None:
        rows[inject[0], inject[1]] = 0x7C00
    return rows


@pytest.mark.parametrize("max_norm", [1e-3, 1e9])
def test_dynamic_scale_and_clipping_bitwise(max_norm):
    n_dp, numel, micro, steps = 4, 40_000, 2, 7
    growth, backoff, interval = 2.0, 0.5, 3
    cfg = 120
    lay, ranks = _group(n_dp, numel, cfg)
    s = lay.shard
    dls = zs.new_loss_scale(65536.0)
    o_scale = np.array([65536.0], np.float32)
    o_good = np.zeros(1, np.int32)
    wf = torch.zeros(lay.n_pad, dtype=torch.bfloat16, device="cuda")
    wout = np.zeros(lay.n_pad, np.uint16)
    overflow_steps = {3: (1, 2, 17), 4: (0, 0, s - 1)}  # step -> (rank, row, element)
    for t in range(1, steps + 1):
        scale_now = float(o_scale[0])
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        o_flag = np.zeros(1, np.uint32)
        part = torch.zeros(n_dp, dtype=torch.float64, device="cuda")
        o_ss = 0.0
        for r, st in enumerate(ranks):
            for mb in range(micro):
                inj = overflow_steps.get(t)
                inj = (inj[1], inj[2]) if inj and inj[0] == r and mb == micro - 1 else None
                rows = _rows(cfg, t, mb, n_dp, r * s, s, numel, scale_now, inj)
                last = mb == micro - 1
                zs.zero_shard_reduce(dev16(rows, zs.ZERO_FP16), n_dp, s, s, st["dacc"],
                                     accumulate=mb > 0, overflow=flag,
                                     sumsq=part[r:r + 1] if last else None)
                o_part = np.zeros(1, np.float64)
                oracle.reduce(rows, oracle.FP16, n_dp, s, s, st["acc"], mb > 0, overflow=o_flag,
                              sumsq=o_part if last else None)
                if last:
                    o_ss += float(o_part[0])
        torch.cuda.synchronize()
        assert int(flag.item()) == int(o_flag[0])
        if np.isfinite(o_ss):
            assert abs(float(part.sum().item()) - o_ss) <= 1e-10 * o_ss
        d_ss = torch.tensor([o_ss], dtype=torch.float64, device="cuda")
        hp = zs.AdamWHParams(step=t, grad_scale=1.0 / (n_dp * micro), **HP)
        for r, st in enumerate(ranks):
            zs.zero_shard_adamw_ex(st["dacc"], st["dw"], st["dm"], st["dv"], wf, lay, r, hp,
                                   skip=flag, sumsq=d_ss, max_norm=max_norm, loss_scale=dls)
            slot = wout[r * s:(r + 1) * s].copy()
            oracle.adamw_ex(st["acc"], st["w"], st["m"], st["v"], slot, oracle.BF16, s, t,
                            grad_scale=1.0 / (n_dp * micro), skip=o_flag,
                            sumsq=np.array([o_ss]), max_norm=max_norm, loss_scale=o_scale, **HP)
            wout[r * s:(r + 1) * s] = slot
        zs.zero_loss_scale_update(dls, flag, growth, backoff, interval)
        oracle.loss_scale_update(o_scale, o_good, int(o_flag[0]), growth, backoff, interval)
        torch.cuda.synchronize()
        assert zs.read_loss_scale(dls) == (float(o_scale[0]), int(o_good[0])), f"t={t}"
        for st in ranks:
            diff = check_f32(hostf(st["dacc"]), st["acc"], "acc")
            diff += check_f32(hostf(st["dw"]), st["w"], "master") + check_f32(hostf(st["dm"]), st["m"], "m")
            diff += check_f32(hostf(st["dv"]), st["v"], "v")
            assert diff == 0, f"t={t}"
        assert check_16(host16(wf), wout, 0, "weights") == 0
    # the injected overflows skipped two steps and backed the scale off twice
    assert float(o_scale[0]) < 65536.0 * 2


def test_device_clip_coefficient_matches_host():
    """The device computes c = min(1, max_norm / (sqrt(sumsq) * s + 1e-6)) in
    double; over many sums its choice equals the host's, bit for bit."""
    lay, _ = zs.zero_flatten_layout([8], 1, 8)
    rng = np.random.default_rng(5)
    acc = np.full(8, 1.0, np.float32)
    dacc = devf(acc)
    vals = np.exp(rng.uniform(np.log(1e-8), np.log(1e8), size=300))
    dss = torch.tensor(vals, dtype=torch.float64, device="cuda")
    outs = torch.zeros((vals.size, 8), dtype=torch.float32, device="cuda")
    wf = torch.zeros(8, dtype=torch.bfloat16, device="cuda")
    hp = zs.AdamWHParams(step=1, grad_scale=0.25, lr=1e-2, weight_decay=0.0)
    for i in range(vals.size):
        dm = torch.zeros(8, device="cuda")
        dv = torch.zeros(8, device="cuda")
        zs.zero_shard_adamw_ex(dacc, outs[i], dm, dv, wf, lay, 0, hp, sumsq=dss[i:i + 1],
                               max_norm=1.0)
        # m = 0.1 * g * c exposes the coefficient: compare with the host's m
        outs[i].copy_(dm)
    got = outs.cpu().numpy()
    for i, x in enumerate(vals):
        w, m, v, wo = np.zeros(8, np.float32), np.zeros(8, np.float32), np.zeros(8, np.float32), np.zeros(8, np.uint16)
        oracle.adamw_ex(acc, w, m, v, wo, oracle.BF16, 8, 1, lr=1e-2, beta1=0.9, beta2=0.999,
                        eps=1e-8, weight_decay=0.0, grad_scale=0.25, sumsq=np.array([x]),
                        max_norm=1.0)
        assert np.array_equal(got[i].view(np.uint32), m.view(np.uint32)), f"sumsq={x}"


def test_all_gpu_pipeline_within_bar():
    """Everything on the device (the ranks' partial sums added on the device
    too): within the stated bar of the oracle run with its own sums."""
    n_dp, numel, micro = 2, 30_000, 2
    cfg = 121
    lay, ranks = _group(n_dp, numel, cfg)
    s = lay.shard
    dls = zs.new_loss_scale(65536.0)
    o_scale = np.array([65536.0], np.float32)
    o_good = np.zeros(1, np.int32)
    wf = torch.zeros(lay.n_pad, dtype=torch.bfloat16, device="cuda")
    wout = np.zeros(lay.n_pad, np.uint16)
    for t in range(1, 4):
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        part = torch.zeros(n_dp, dtype=torch.float64, device="cuda")
        o_flag = np.zeros(1, np.uint32)
        o_ss = 0.0
        for r, st in enumerate(ranks):
            for mb in range(micro):
                rows = _rows(cfg, t, mb, n_dp, r * s, s, numel, float(o_scale[0]), None)
                last = mb == micro - 1
                zs.zero_shard_reduce(dev16(rows, zs.ZERO_FP16), n_dp, s, s, st["dacc"],
                                     accumulate=mb > 0, overflow=flag,
                                     sumsq=part[r:r + 1] if last else None)
                o_part = np.zeros(1, np.float64)
                oracle.reduce(rows, oracle.FP16, n_dp, s, s, st["acc"], mb > 0, overflow=o_flag,
                              sumsq=o_part if last else None)
                o_ss += float(o_part[0]) if last else 0.0
        total = part.sum().reshape(1)
        hp = zs.AdamWHParams(step=t, grad_scale=1.0 / (n_dp * micro), **HP)
        for r, st in enumerate(ranks):
            zs.zero_shard_adamw_ex(st["dacc"], st["dw"], st["dm"], st["dv"], wf, lay, r, hp,
                                   skip=flag, sumsq=total, max_norm=1e-3, loss_scale=dls)
            slot = wout[r * s:(r + 1) * s].copy()
            oracle.adamw_ex(st["acc"], st["w"], st["m"], st["v"], slot, oracle.BF16, s, t,
                            grad_scale=1.0 / (n_dp * micro), skip=o_flag, sumsq=np.array([o_ss]),
                            max_norm=1e-3, loss_scale=o_scale, **HP)
            wout[r * s:(r + 1) * s] = slot
        zs.zero_loss_scale_update(dls, flag, 2.0, 0.5, 2)
        oracle.loss_scale_update(o_scale, o_good, int(o_flag[0]), 2.0, 0.5, 2)
    torch.cuda.synchronize()
    for st in ranks:
        check_f32(hostf(st["dw"]), st["w"], "master")
        check_f32(hostf(st["dm"]), st["m"], "m")
        check_f32(hostf(st["dv"]), st["v"], "v")
    check_16(host16(wf), wout, 0, "weights", max_ulp=1)
    assert zs.read_loss_scale(dls) == (float(o_scale[0]), int(o_good[0]))
