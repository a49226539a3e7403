"""Pins of the oracle's step controls (CPU only): global-norm gradient
clipping (gradient clipping 1.0 in the configs of "DeepSpeed ZeRO", "A
worked example", and "ZeRO Optimizer, in depth", "Running it with
DeepSpeed") and the dynamic fp16 loss scale ("DeepSpeed ZeRO", "Mixed
precision").  References: torch's loss-scale update op and
torch.nn.utils.clip_grad_norm_ with torch.optim.AdamW (library routines),
and closed forms."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import F32, tag

HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
U = 2.0 ** -24


@pytest.mark.parametrize("growth,backoff,interval", [(2.0, 0.5, 7), (2.0, 0.5, 1), (1.5, 0.7, 4)])
def test_loss_scale_matches_torch(growth, backoff, interval):
    rng = np.random.default_rng(interval)
    ovf = (rng.random(300) < 0.15).astype(np.uint32)
    s = np.array([65536.0], np.float32)
    g = np.zeros(1, np.int32)
    ts = torch.tensor([65536.0])
    tg = torch.tensor([0], dtype=torch.int32)
    for o in ovf:
        oracle.loss_scale_update(s, g, o, growth, backoff, interval)
        torch._amp_update_scale_(ts, tg, torch.tensor([float(o)]), growth, backoff, interval)
        assert s[0] == ts.item() and g[0] == tg.item()


def test_loss_scale_closed_form():
    s = np.array([65536.0], np.float32)
    g = np.zeros(1, np.int32)
    for _ in range(3 * 5):  # 15 good steps at interval 5: three doublings
        oracle.loss_scale_update(s, g, 0, 2.0, 0.5, 5)
    assert s[0] == 65536.0 * 8 and g[0] == 0
    oracle.loss_scale_update(s, g, 1, 2.0, 0.5, 5)
    assert s[0] == 65536.0 * 4 and g[0] == 0


def _vec(n, seed, sigma):
    return synth.fill_host(F32, seed, tag(5, 60), 0, n, sigma)


@pytest.mark.parametrize("max_norm", [0.05, 1.0, 100.0])
def test_clip_coefficient_matches_torch(max_norm):
    g = _vec(50_000, 1, 1e-2)  # norm about 2.2
    c = oracle.clip_coef(float(np.sum(g.astype(np.float64) ** 2)), 1.0, max_norm)
    p = torch.nn.Parameter(torch.zeros(g.size))
    p.grad = torch.from_numpy(g.copy())
    torch.nn.utils.clip_grad_norm_([p], max_norm, foreach=False)
    ref = p.grad.numpy()
    ours = (g * np.float32(c)).astype(np.float32) if c < 1 else g
    assert np.allclose(ours, ref, rtol=1e-6, atol=0)
    if c < 1:  # the clipped gradient has norm max_norm
        assert abs(np.sqrt(np.sum(ours.astype(np.float64) ** 2)) - max_norm) <= 1e-6 * max_norm
    else:
        assert c == 1.0


def test_clipped_adamw_matches_torch():
    n, steps, max_norm = 4096, 6, 0.01
    w, m, v = _vec(n, 2, 0.02), np.zeros(n, np.float32), np.zeros(n, np.float32)
    wout = np.zeros(n, np.uint16)
    p = torch.nn.Parameter(torch.from_numpy(w.copy()))
    opt = torch.optim.AdamW([p], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=HP["weight_decay"], foreach=False)
    mag = np.zeros(n)
    for t in range(1, steps + 1):
        acc = synth.fill_host(F32, 3, tag(5, 61, t), 0, n, 1e-3)
        ss = np.array([np.sum(acc.astype(np.float64) ** 2)])
        oracle.adamw_ex(acc, w, m, v, wout, oracle.BF16, n, t, sumsq=ss, max_norm=max_norm, **HP)
        p.grad = torch.from_numpy(acc.copy())
        torch.nn.utils.clip_grad_norm_([p], max_norm, foreach=False)
        opt.step()
        st = opt.state[p]
        gx = np.abs(p.grad.numpy()).astype(np.float64)
        mag = HP["beta1"] * mag + (1 - HP["beta1"]) * gx
        assert np.all(np.abs(m - st["exp_avg"].numpy()) <= 16 * U * mag * t)
        assert np.all(np.abs(v - st["exp_avg_sq"].numpy()) <= 16 * U * st["exp_avg_sq"].numpy() * t)
        tw = p.detach().numpy()
        assert np.all(np.abs(w - tw) <= t * (4 * U * np.abs(tw) + HP["lr"] * 2e-6))


def test_controls_reduce_to_plain_adamw_bitwise():
    n = 3000
    acc = _vec(n, 4, 1e-3)
    base = [_vec(n, 5, 0.02), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)]
    plain = [x.copy() for x in base]
    oracle.adamw(acc, *plain, oracle.BF16, n, 2, grad_scale=1.0 / (8 * 65536 * 4), **HP)
    # inactive clipping and a dynamic loss scale equal to the static one
    ex = [x.copy() for x in base]
    oracle.adamw_ex(acc, *ex, oracle.BF16, n, 2, grad_scale=1.0 / (8 * 4),
                    loss_scale=np.array([65536.0], np.float32),
                    sumsq=np.array([1e-12]), max_norm=1.0, **HP)
    for a, b in zip(plain, ex):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    # skip writes nothing
    sk = [x.copy() for x in base]
    oracle.adamw_ex(acc, *sk, oracle.BF16, n, 2, skip=np.ones(1, np.uint32), sumsq=np.array([1.0]),
                    max_norm=1e-3, **HP)
    for a, b in zip(base, sk):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_clipping_scales_the_step_1_update():
    """At t = 1 Adam's update is ~lr * sign(g) whatever the gradient's size,
    so clipping must leave step 1's master unchanged up to eps effects while
    m holds the clipped gradient: m_1 = 0.1 * c * g."""
    n = 2048
    acc = _vec(n, 6, 1.0)
    ss = np.array([np.sum(acc.astype(np.float64) ** 2)])
    c = oracle.clip_coef(ss[0], 1.0, 1.0)
    assert 0 < c < 0.05
    w, m, v, wo = _vec(n, 7, 0.02), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    oracle.adamw_ex(acc, w, m, v, wo, oracle.BF16, n, 1, sumsq=ss, max_norm=1.0, **HP)
    g = acc.astype(np.float64) * c
    assert np.all(np.abs(m - 0.1 * g) <= 4 * U * 0.1 * np.abs(g))


def test_clip_norm_is_of_the_unscaled_gradient():
    """The norm compared with max_norm is that of g = acc * s, not of the
    loss-scaled accumulator: clipping a loss-scaled accumulator (s = 2^-19)
    gives exactly what clipping the unscaled gradient (s = 1) gives."""
    n, s = 4096, 2.0 ** -19
    g = _vec(n, 8, 1e-2)
    acc = (g.astype(np.float64) / s).astype(np.float32)  # exact: power of two
    out = []
    for a, gs in ((g, 1.0), (acc, s)):
        w, m, v, wo = _vec(n, 9, 0.02), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
        ss = np.array([np.sum(a.astype(np.float64) ** 2)])
        oracle.adamw_ex(a, w, m, v, wo, oracle.BF16, n, 1, grad_scale=gs, sumsq=ss, max_norm=0.5, **HP)
        out.append((w, m, v))
    for x, y in zip(*out):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert oracle.clip_coef(float(np.sum(acc.astype(np.float64) ** 2)), s, 0.5) < 1.0
