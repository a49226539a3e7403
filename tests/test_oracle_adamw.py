"""Pins of the oracle's AdamW update on the owned shard (CPU only).

"ZeRO and FSDP" (Zero to Frontier 10.3), "A sharded Adam step": Adam with
bias correction from t = 1 on each rank's own shard; the configs of
"DeepSpeed ZeRO" ("A worked example") and "ZeRO Optimizer, in depth"
("Running it with DeepSpeed") name AdamW, read as decoupled weight decay.
The pins are independent of the oracle's own code: torch.optim.AdamW and
torch.optim.Adam (library routines), closed forms, a high-precision brute
force with a derived rounding bound, and invariants the pages state.
"""
import decimal
from decimal import Decimal as D

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import BF16, F16, F32, tag
from synth.synth_const import BUF_GRAD, BUF_MASTER
from tests.util import ulp_diff

HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
U = 2.0 ** -24


def _grads(n, length, step, cfg, kind=BF16, sigma=1e-3, thr=0, mul=1.0):
    return np.stack([synth.fill_host(kind, 0, tag(BUF_GRAD, cfg, step, 0, k), 0, length,
                                     sigma, thr, mul) for k in range(n)])


def _master(length, cfg):
    return synth.fill_host(F32, 0, tag(BUF_MASTER, cfg), 0, length, 0.02)


def _state(length, cfg):
    return (_master(length, cfg), np.zeros(length, np.float32), np.zeros(length, np.float32),
            np.zeros(length, np.uint16))


# ---------------------------------------------------------------------------
# library routines


@pytest.mark.parametrize("wd", [0.1, 0.0])
def test_matches_torch_adamw_single_rank(wd):
    """n_dp = 1: the reduce is the identity, the step is torch's AdamW (or
    Adam when wd = 0).  torch groups the bias corrections differently, so
    the comparison is within a rounding tolerance, not bitwise."""
    length, steps = 4096, 10
    hp = dict(HP, weight_decay=wd)
    w, m, v, wout = _state(length, 50)
    p = torch.nn.Parameter(torch.from_numpy(w.copy()))
    if wd:
        opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]),
                                eps=hp["eps"], weight_decay=wd, foreach=False)
    else:
        opt = torch.optim.Adam([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]),
                               eps=hp["eps"], foreach=False)
    mag = np.zeros(length)  # running sum of |terms| that make up m
    for t in range(1, steps + 1):
        g = _grads(1, length, t, 50, thr=synth.outlier_threshold(0.01), mul=100.0)
        oracle.step(g, oracle.BF16, 1, length, length, w, m, v, wout, oracle.BF16, t, **hp)
        p.grad = torch.from_numpy(oracle.bf16_to_f32(g[0]))
        opt.step()
        st = opt.state[p]
        tm, tv, tw = st["exp_avg"].numpy(), st["exp_avg_sq"].numpy(), p.detach().numpy()
        gx = np.abs(oracle.bf16_to_f32(g[0])).astype(np.float64)
        mag = hp["beta1"] * mag + (1 - hp["beta1"]) * gx
        # M: lerp vs b1*m + c1*g, a few roundings per step on terms whose
        # magnitudes sum to mag (m itself may cancel)
        assert np.all(np.abs(m - tm) <= 8 * U * mag * t)
        assert np.all(np.abs(v - tv) <= 8 * U * np.abs(tv) * t)
        # W: a few ulps of W per step plus a relative 1e-6 of each update
        assert np.all(np.abs(w - tw) <= t * (4 * U * np.abs(tw) + hp["lr"] * 1e-6))
    # the 16-bit weights are the RNE cast of the master
    ref16 = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wout, ref16)


@pytest.mark.parametrize("n_dp", [1, 3, 8])
def test_matches_a_numpy_transcription_of_the_pages_sharded_step(n_dp):
    """"ZeRO and FSDP", A sharded Adam step, written out in NumPy float32 from
    its prose: the ranks' gradients averaged (summed over ranks in order,
    divided by n_dp), Adam with bias correction from t = 1 on the whole
    vector -- the pieces of numpy.array_split updated independently are
    the same update.  The constants are formed as the stated reading does
    (in double, rounded once; beta^t from the C library's pow through
    Python) and the update grouped as documented, lr * (mhat / (sqrt(vhat)
    + eps)).  Independent code, the same rounding at each operation: the
    oracle's reduce and AdamW per piece (wd = 0, grad_scale = fl(1/n_dp))
    must agree bit for bit wherever fl(1/n_dp) is exact (n_dp = 1, 8), and
    for n_dp = 3 -- where dividing and multiplying by the rounded reciprocal
    differ in the last bit -- within a few roundings."""
    n, steps = 5003, 5
    lr, b1, b2, eps = 1e-3, 0.9, 0.999, 1e-8
    f32 = np.float32
    w0 = _master(n, 59)
    W, Mn, Vn = w0.copy(), np.zeros(n, f32), np.zeros(n, f32)
    pieces = np.array_split(np.arange(n), n_dp)
    ow = [w0[p].copy() for p in pieces]
    om = [np.zeros(p.size, f32) for p in pieces]
    ov = [np.zeros(p.size, f32) for p in pieces]
    c1, c2 = f32(1.0 - b1), f32(1.0 - b2)
    mag = np.zeros(n)  # running sum of |terms| that make up m (m itself may cancel)
    for t in range(1, steps + 1):
        bc1, bc2 = f32(1.0 - b1 ** t), f32(1.0 - b2 ** t)
        rows = _grads(n_dp, n, t, 59)
        x = oracle.bf16_to_f32(rows)
        G = x[0].copy()
        for k in range(1, n_dp):
            G = (G + x[k]).astype(f32)
        G = (G / f32(n_dp)).astype(f32)
        mag = b1 * mag + (1 - b1) * np.abs(G.astype(np.float64))
        Mn = (f32(b1) * Mn + c1 * G).astype(f32)
        Vn = (f32(b2) * Vn + c2 * (G * G)).astype(f32)
        mhat, vhat = (Mn / bc1).astype(f32), (Vn / bc2).astype(f32)
        W = (W - f32(lr) * (mhat / (np.sqrt(vhat) + f32(eps)))).astype(f32)
        for r, p in enumerate(pieces):
            if p.size == 0:
                continue
            acc = np.zeros(p.size, f32)
            oracle.reduce(np.ascontiguousarray(rows[:, p]), oracle.BF16, n_dp, p.size, p.size,
                          acc, 0)
            wo = np.zeros(p.size, np.uint16)
            oracle.adamw(acc, ow[r], om[r], ov[r], wo, oracle.BF16, p.size, t, lr=lr, beta1=b1,
                         beta2=b2, eps=eps, weight_decay=0.0, grad_scale=1.0 / n_dp)
        w, m, v = np.concatenate(ow), np.concatenate(om), np.concatenate(ov)
        if n_dp in (1, 8):
            for a, b in ((w, W), (m, Mn), (v, Vn)):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"t={t}"
        else:
            # g differs by at most an ulp; m and v carry it (a few roundings
            # per step), the update by a relative few ulps
            assert np.all(np.abs(m - Mn) <= 8 * U * t * mag)
            assert np.all(np.abs(v - Vn) <= 8 * U * t * np.abs(Vn) + 1e-30)
            assert np.all(np.abs(w - W) <= t * (4 * U * np.abs(W) + lr * 1e-6))


# ---------------------------------------------------------------------------
# closed forms


def test_step1_update_is_lr_times_sign():
    """At t = 1 with m = v = 0: mhat = g, vhat = g^2, so the Adam part of the
    update is lr * g / (|g| + eps) ~ lr * sign(g); decoupled decay adds
    -lr * wd * w."""
    length, n = 8192, 4
    rows = _grads(n, length, 1, 51)
    w, m, v, wout = _state(length, 51)
    w0 = w.copy()
    oracle.step(rows, oracle.BF16, n, length, length, w, m, v, wout, oracle.BF16, 1, **HP)
    g = oracle.bf16_to_f32(rows).astype(np.float64).sum(0) / n
    lr, wd, eps = HP["lr"], HP["weight_decay"], HP["eps"]
    ref = w0 - lr * wd * w0 - lr * np.sign(g)
    bound = lr * eps / (np.abs(g) + eps) + lr * 1e-6 + 3 * U * 2 * np.abs(w0)
    assert np.all(np.abs(w - ref) <= bound)
    assert np.all(np.sign(w0 - w - lr * wd * w0)[g != 0] == np.sign(g[g != 0]))


def test_constant_gradient_closed_form():
    """With the same g every step, exact Adam has mhat_t = g and vhat_t = g^2
    for all t, so W_t = W_0 d^t - lr u sum_{i<t} d^i, u = g / (|g| + eps),
    d = 1 - lr wd."""
    length, n, steps = 4096, 2, 10
    rows = _grads(n, length, 1, 52)
    w, m, v, wout = _state(length, 52)
    w0 = w.astype(np.float64)
    for t in range(1, steps + 1):
        oracle.step(rows, oracle.BF16, n, length, length, w, m, v, wout, oracle.BF16, t, **HP)
    g = oracle.bf16_to_f32(rows).astype(np.float64).sum(0) / n
    lr, wd, eps = HP["lr"], HP["weight_decay"], HP["eps"]
    d = 1.0 - lr * wd
    u = g / (np.abs(g) + eps)
    wt = w0 * d ** steps - lr * u * sum(d ** i for i in range(steps))
    bound = steps * (4 * U * np.abs(wt) + lr * 1e-5)
    assert np.all(np.abs(w - wt) <= bound)
    mt = g * (1 - HP["beta1"] ** steps)
    assert np.all(np.abs(m - mt) <= steps * 4 * U * np.abs(g))


# ---------------------------------------------------------------------------
# brute force in high precision with a derived rounding bound


decimal.getcontext().prec = 50


def _exact_step(x16, gdt, n, M, V, W, t, hp):
    """One step in 50-digit decimal from the given fp32 state and 16-bit rows,
    with the real (unrounded) hyperparameters.  Returns the exact results
    and first-order bounds on the oracle's rounding errors."""
    xs = [D(float(v)) for v in x16]
    lr, b1, b2 = D(repr(hp["lr"])), D(repr(hp["beta1"])), D(repr(hp["beta2"]))
    eps, wd = D(repr(hp["eps"])), D(repr(hp["weight_decay"]))
    u = D(2) ** -24
    M, V, W = D(float(M)), D(float(V)), D(float(W))
    G = sum(xs) / n
    eG = (n - 1) * u * sum(abs(x) for x in xs) / n + u * abs(G)
    Ms = b1 * M + (1 - b1) * G
    eM = (1 - b1) * eG * (1 + u) + 4 * u * (b1 * abs(M) + (1 - b1) * abs(G))
    Vs = b2 * V + (1 - b2) * G * G
    eV = (1 - b2) * (2 * abs(G) * eG + eG * eG) + 5 * u * (b2 * V + (1 - b2) * G * G)
    bc1, bc2 = 1 - b1 ** t, 1 - b2 ** t
    mh, vh = Ms / bc1, Vs / bc2
    emh = eM / bc1 * (1 + 2 * u) + 2 * u * abs(mh)
    evh = eV / bc2 * (1 + 2 * u) + 2 * u * vh
    sq = vh.sqrt()
    esq = sq - max(D(0), vh - evh).sqrt() + 2 * u * sq
    den = sq + eps
    eden = esq + u * den + 2 * u * eps
    us = mh / den
    dmin = den - eden
    eu = emh / dmin + abs(mh) * eden / (den * dmin) + u * abs(us)
    Ws = W * (1 - lr * wd) - lr * us
    eW = 3 * u * abs(W) + lr * eu * (1 + u) + 3 * u * lr * abs(us) + u * abs(Ws)
    return (Ms, eM), (Vs, eV), (Ws, eW)


@pytest.mark.parametrize("n,gdt", [(1, oracle.BF16), (3, oracle.BF16), (8, oracle.BF16),
                                   (4, oracle.FP16)])
def test_brute_force_high_precision_tiny(n, gdt):
    length, steps = 24, 10
    kind, sigma = (BF16, 1e-3) if gdt == oracle.BF16 else (F16, 1e-3)
    w, m, v, wout = _state(length, 53 + n)
    for t in range(1, steps + 1):
        rows = _grads(n, length, t, 53 + n, kind, sigma, thr=synth.outlier_threshold(0.1),
                      mul=100.0)
        x = oracle.f16_to_f32(rows) if gdt == oracle.FP16 else oracle.bf16_to_f32(rows)
        prev = (m.copy(), v.copy(), w.copy())
        oracle.step(rows, gdt, n, length, length, w, m, v, wout, oracle.BF16, t, **HP)
        for j in range(length):
            (Ms, eM), (Vs, eV), (Ws, eW) = _exact_step(x[:, j], gdt, n, prev[0][j], prev[1][j],
                                                       prev[2][j], t, HP)
            assert abs(D(float(m[j])) - Ms) <= 2 * eM, (t, j, "m")
            assert abs(D(float(v[j])) - Vs) <= 2 * eV, (t, j, "v")
            assert abs(D(float(w[j])) - Ws) <= 2 * eW, (t, j, "w")
        assert np.all(v >= 0)


# ---------------------------------------------------------------------------
# invariants the pages state


def test_sharded_update_equals_unsharded():
    """Every rank updating its own shard and all-gathering gives exactly the
    update one rank would make on the whole vector with the all-reduced
    gradient ("ZeRO and FSDP": sixty-three of 64 redundant updates are waste,
    and removing them changes nothing)."""
    n_dp, numels = 8, [5000, 3, 1234, 777]
    _, n, n_pad, s = oracle.flatten_layout(numels, n_dp)
    full = _grads(n_dp, n_pad, 1, 55, thr=synth.outlier_threshold(0.01), mul=100.0)
    full[:, n:] = 0
    W0 = _master(n_pad, 55)
    W0[n:] = 0
    # unsharded: one "rank" holding everything
    wu, mu, vu = W0.copy(), np.zeros(n_pad, np.float32), np.zeros(n_pad, np.float32)
    bu = np.zeros(n_pad, np.uint16)
    # sharded: rank r owns [r s, (r + 1) s), writes its slot of the full buffer
    ws, ms, vs = W0.copy(), np.zeros(n_pad, np.float32), np.zeros(n_pad, np.float32)
    bs = np.full(n_pad, 0xBEEF, np.uint16)
    flat = full.reshape(-1)
    for t in (1, 2, 3):
        oracle.step(full, oracle.BF16, n_dp, n_pad, n_pad, wu, mu, vu, bu, oracle.BF16, t,
                    grad_scale=1.0 / n_dp, **HP)
        for r in range(n_dp):
            sl = slice(r * s, (r + 1) * s)
            w_, m_, v_, b_ = ws[sl].copy(), ms[sl].copy(), vs[sl].copy(), bs[sl].copy()
            oracle.step(np.ascontiguousarray(flat[r * s:]), oracle.BF16, n_dp, n_pad, s,
                        w_, m_, v_, b_, oracle.BF16, t, **HP)
            ws[sl], ms[sl], vs[sl], bs[sl] = w_, m_, v_, b_
        for a, b in ((wu, ws), (mu, ms), (vu, vs)):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        assert np.array_equal(bu, bs)
    # padding stays exactly +0
    assert np.all(ws[n:].view(np.uint32) == 0) and np.all(bs[n:] == 0)


def test_fused_equals_reduce_then_adamw():
    n, length = 8, 3000
    rows = _grads(n, length, 1, 56, F16, 65.536)
    s = 1.0 / (n * 65536.0)
    a = _state(length, 56)
    b = tuple(x.copy() for x in a)
    oracle.step(rows, oracle.FP16, n, length, length, *a, oracle.BF16, 3, grad_scale=s, **HP)
    acc = np.zeros(length, np.float32)
    oracle.reduce(rows, oracle.FP16, n, length, length, acc, 0)
    oracle.adamw(acc, *b, oracle.BF16, length, 3, grad_scale=s, **HP)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("n", [1, 3, 8])
def test_step_sum_of_squares_and_flag(n):
    """The fused step's shard-wide reductions: the sum of squares is that of
    the averaged gradient g = fl(a * s), a the left-to-right fp32 sum of the
    rows (computed here with numpy), checked in float64; the overflow flag is
    raised by a non-finite row element and only then."""
    length = 3000
    rows = _grads(n, length, 1, 58, BF16, thr=10486, mul=100.0)
    x = oracle.bf16_to_f32(rows)
    a = x[0].copy()
    for k in range(1, n):
        a = (a + x[k]).astype(np.float32)
    g = (a * np.float32(1.0 / n)).astype(np.float32)
    ss, flag = np.zeros(1), np.zeros(1, np.uint32)
    oracle.step(rows, oracle.BF16, n, length, length, *_state(length, 58), oracle.BF16, 1,
                grad_scale=1.0 / n, overflow=flag, sumsq=ss, **HP)
    ref = np.sum(g.astype(np.float64) ** 2)
    assert flag[0] == 0 and abs(ss[0] - ref) <= 1e-12 * ref
    rows[n - 1, 1234] = 0xFF80  # -inf in the last row
    oracle.step(rows, oracle.BF16, n, length, length, *_state(length, 58), oracle.BF16, 1,
                grad_scale=1.0 / n, overflow=flag, **HP)
    assert flag[0] == 1


def test_skip_flag_leaves_state_untouched():
    length = 1000
    acc = np.ones(length, np.float32)
    w, m, v, wout = _state(length, 57)
    snap = [x.copy() for x in (w, m, v, wout)]
    oracle.adamw(acc, w, m, v, wout, oracle.BF16, length, 1,
                 skip=np.ones(1, np.uint32), **HP)
    for x, y in zip((w, m, v, wout), snap):
        assert np.array_equal(x, y)
    oracle.adamw(acc, w, m, v, wout, oracle.BF16, length, 1,
                 skip=np.zeros(1, np.uint32), **HP)
    assert not np.array_equal(w, snap[0])


def test_snapshot_and_resume_is_bit_identical():
    n, length = 4, 2048
    w, m, v, wout = _state(length, 58)
    traj = []
    snap = None
    for t in range(1, 7):
        oracle.step(_grads(n, length, t, 58), oracle.BF16, n, length, length, w, m, v, wout,
                    oracle.BF16, t, **HP)
        if t == 3:
            snap = [x.copy() for x in (w, m, v)]
        traj.append(w.copy())
    w2, m2, v2 = snap
    b2 = np.zeros(length, np.uint16)
    for t in range(4, 7):
        oracle.step(_grads(n, length, t, 58), oracle.BF16, n, length, length, w2, m2, v2, b2,
                    oracle.BF16, t, **HP)
    assert np.array_equal(w2.view(np.uint32), traj[-1].view(np.uint32))


def test_fp16_weight_output_is_the_rne_cast():
    length = 2048
    rows = _grads(2, length, 1, 59)
    w, m, v, wout = _state(length, 59)
    oracle.step(rows, oracle.BF16, 2, length, length, w, m, v, wout, oracle.FP16, 1, **HP)
    ref = torch.from_numpy(w).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wout, ref)


def test_scalars_follow_the_stated_rounding():
    c = oracle.adamw_scalars(1, **HP)
    assert c["c1"] == np.float32(0.1) and c["c2"] == np.float32(0.001)
    assert c["bc1"] == np.float32(1 - 0.9) and c["bc2"] == np.float32(1 - 0.999)
    assert c["d"] == np.float32(1 - 1e-5)
    c10 = oracle.adamw_scalars(10, **HP)
    assert ulp_diff(np.float32(c10["bc1"]), np.float32(1 - 0.9 ** 10))[()] == 0


@pytest.mark.parametrize("t,grad_scale", [(1, 0.125), (7, 1.0 / 3.0)])
def test_each_operation_is_one_binary32_rounding(t, grad_scale):
    """The oracle's update is the stated sequence of binary32 operations,
    each rounded once to nearest-even (no contraction, no reassociation, no
    reciprocal in place of a division): every element re-derived here in
    exact rational arithmetic with one rounding per operation equals the
    oracle's bits.  The constants are formed in double from the double
    hyperparameters and rounded once (b1 = fl(beta1), c1 = fl(1 - beta1),
    bc1 = fl(1 - beta1^t), d = fl(1 - lr * wd), s = fl(grad_scale)).  The
    square root is the correctly rounded double sqrt rounded to binary32:
    double has more than 2 * 24 + 2 bits, so that second rounding gives the
    correctly rounded binary32 root (Figueroa, "When is double rounding
    innocuous?", 1995)."""
    import math
    from fractions import Fraction as Fr
    from tests.util import rne_f32
    n = 400
    rng = np.random.default_rng(100 + t)
    acc = (rng.standard_normal(n) * 8e-3).astype(np.float32)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = ((rng.standard_normal(n) * 1e-3) ** 2).astype(np.float32) + np.float32(1e-12)
    hp = dict(HP)
    f32 = lambda x: Fr(float(np.float32(x)))          # one rounding from double
    b1, c1 = f32(hp["beta1"]), f32(1.0 - hp["beta1"])
    b2, c2 = f32(hp["beta2"]), f32(1.0 - hp["beta2"])
    bc1, bc2 = f32(1.0 - math.pow(hp["beta1"], t)), f32(1.0 - math.pow(hp["beta2"], t))
    lr, eps = f32(hp["lr"]), f32(hp["eps"])
    d, s = f32(1.0 - hp["lr"] * hp["weight_decay"]), f32(grad_scale)
    R = rne_f32
    want_w, want_m, want_v = [], [], []
    for j in range(n):
        g = R(Fr(float(acc[j])) * s)
        mt = R(R(b1 * Fr(float(m[j]))) + R(c1 * g))
        vt = R(R(b2 * Fr(float(v[j]))) + R(c2 * R(g * g)))
        mhat, vhat = R(mt / bc1), R(vt / bc2)
        root = Fr(float(np.float32(math.sqrt(float(vhat)))))
        den = R(root + eps)
        u = R(mhat / den)
        wt = R(R(Fr(float(w[j])) * d) - R(lr * u))
        want_w.append(float(wt))
        want_m.append(float(mt))
        want_v.append(float(vt))
    wout = np.zeros(n, np.uint16)
    oracle.adamw(acc, w, m, v, wout, oracle.BF16, n, t, grad_scale=grad_scale, **hp)
    assert np.array_equal(w.view(np.uint32), np.array(want_w, np.float32).view(np.uint32))
    assert np.array_equal(m.view(np.uint32), np.array(want_m, np.float32).view(np.uint32))
    assert np.array_equal(v.view(np.uint32), np.array(want_v, np.float32).view(np.uint32))
