"""GPU parity of the HIP path (called through the C ABI) against the CPU
oracle, element by element, on seeded inputs at sizes the oracle finishes in
seconds: the tiny workload, mid sizes spanning many tiles with ragged tails,
every rank, both 16-bit formats, buckets, accumulation, the overflow gate.

The bar: layout, indexing, padding and untouched bytes bit-exact; fp32
master/m/v within max relative error 1e-6; 16-bit weights within 1 ulp.
The arithmetic follows one fixed order on both sides, so every comparison
also counts (and here requires zero) non-identical elements.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_flatten_amd as zs
from synth.workloads import GradDraw, workload
from synth import BF16, F16
from tests.gpu_util import (check_16, check_f32, dev16, devf, host16, host_master, host_rows,
                            hostf)

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
CANARY = 0x5A5A


def _run_case(numels, n_dp, rank, steps, draw, cfg, wdt=zs.ZERO_BF16, align=1, ld_pad=0,
              sumsq=False, overflow=False, buckets=None):
    """Run `steps` fused steps on the GPU and on the oracle from the same
    seeded inputs; compare everything after every step."""
    lay, _ = zs.zero_flatten_layout(numels, n_dp, align)
    _, n, n_pad, s = oracle.flatten_layout(numels, n_dp, align)
    assert (lay.n, lay.n_pad, lay.shard) == (n, n_pad, s)
    gdt = zs.ZERO_BF16 if draw.kind == BF16 else zs.ZERO_FP16
    lo = rank * s
    ld = s + ld_pad
    w = host_master(cfg, lo, s, pad_from=n)
    m = np.zeros(s, np.float32)
    v = np.zeros(s, np.float32)
    wout = np.full(n_pad, CANARY, np.uint16)
    dw, dm, dv = devf(w), devf(m), devf(v)
    dwf = dev16(wout, wdt)
    dev = torch.device("cuda")
    for t in steps:
        rows = host_rows(cfg, t, 0, n_dp, lo, s, draw, pad_from=n)
        slab = np.zeros((n_dp, ld), np.uint16)
        slab[:, :s] = rows
        dslab = dev16(slab, gdt)
        hp = zs.AdamWHParams(step=t, grad_scale=1.0 / n_dp, **HP)
        d_ovf = torch.zeros(1, dtype=torch.int32, device=dev) if overflow else None
        d_ss = torch.zeros(1, dtype=torch.float64, device=dev) if sumsq else None
        if buckets is None:
            zs.zero_shard_step(dslab, ld, s, dw, dm, dv, dwf, lay, rank, hp,
                               overflow=d_ovf, sumsq=d_ss)
        else:
            for b0, b1 in buckets:
                zs.zero_shard_step(dslab[:, b0:], ld, b1 - b0, dw[b0:], dm[b0:], dv[b0:], dwf,
                                   lay, rank, hp, shard_off=b0, overflow=d_ovf, sumsq=d_ss)
        o_ovf = np.zeros(1, np.uint32)
        o_ss = np.zeros(1, np.float64)
        slot = wout[lo:lo + s].copy()
        oracle.step(np.ascontiguousarray(slab), gdt, n_dp, ld, s, w, m, v, slot, wdt, t,
                    grad_scale=1.0 / n_dp, overflow=o_ovf, sumsq=o_ss, **HP)
        wout[lo:lo + s] = slot
        torch.cuda.synchronize()
        diff = check_f32(hostf(dw), w, f"master t={t}")
        diff += check_f32(hostf(dm), m, f"m t={t}")
        diff += check_f32(hostf(dv), v, f"v t={t}")
        got = host16(dwf)
        diff += check_16(got, wout, wdt, f"weights t={t}")
        assert diff == 0, f"{diff} elements differ from the oracle bitwise at t={t}"
        assert np.array_equal(got[:lo], wout[:lo]) and np.array_equal(got[lo + s:], wout[lo + s:])
        if overflow:
            assert int(d_ovf.item()) == int(o_ovf[0])
        if sumsq:
            ref = float(o_ss[0])
            assert abs(d_ss.item() - ref) <= 1e-10 * ref
    # padding stays exactly +0
    if lo + s > n:
        pad = slice(max(0, n - lo), s)
        assert np.all(hostf(dw)[pad].view(np.uint32) == 0)
        assert np.all(host16(dwf)[max(n, lo):lo + s] == 0)


def test_tiny_workload_all_steps():
    """The tiny workload: 10,000 parameters, 4 ranks, shard 2,500, rank 1,
    steps 1-3 (its slot at byte 5,000 is 8-byte aligned: the vector path)."""
    wl = workload(0)
    _run_case(wl.numels, wl.n_dp, wl.rank, wl.steps, wl.grad, cfg=0)


@pytest.mark.parametrize("rank", [0, 2, 3])
def test_tiny_workload_other_ranks(rank):
    """Rank 3's slot starts at byte 7,500, not 8-byte aligned: the element path."""
    wl = workload(0)
    _run_case(wl.numels, wl.n_dp, rank, (1, 2), wl.grad, cfg=0)


MID = [1 << 20, 13]  # 1,048,589 parameters: many tiles and a ragged tail


@pytest.mark.parametrize("n_dp", [1, 3, 8, 64])
@pytest.mark.parametrize("align", [1, 8])
def test_mid_size(n_dp, align):
    rank = min(1, n_dp - 1)
    draw = GradDraw(BF16, 1e-3, outlier_p=0.01, outlier_mul=100.0)
    _run_case(MID, n_dp, rank, (1, 2, 3), draw, cfg=10 + n_dp, align=align)


@pytest.mark.parametrize("n_dp", [2, 8])
def test_fp16_grads_fp16_weights_last_rank(n_dp):
    draw = GradDraw(F16, 1e-3, scale=65536.0)
    _run_case([333_333, 4096, 7], n_dp, n_dp - 1, (1, 2), draw, cfg=80 + n_dp,
              wdt=zs.ZERO_FP16, align=8)


def test_row_stride_wider_than_shard_and_flags():
    draw = GradDraw(BF16, 1e-3)
    _run_case([200_000], 4, 2, (1, 2, 3, 4), draw, cfg=90, align=8, ld_pad=72,
              sumsq=True, overflow=True)


def test_buckets_equal_one_call():
    draw = GradDraw(BF16, 1e-3)
    numels = [100_000, 28_003]
    s = oracle.flatten_layout(numels, 4, 8)[3]
    buckets = [(0, 4096), (4096, 4101), (4101, 20000), (20000, s)]
    _run_case(numels, 4, 1, (1, 2), draw, cfg=91, align=8, buckets=buckets)


def test_empty_range_is_a_noop():
    lay, _ = zs.zero_flatten_layout([64], 4)
    t = torch.zeros(16, device="cuda")
    g = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    wf = torch.full((64,), 3.0, dtype=torch.bfloat16, device="cuda")
    zs.zero_shard_step(g, 16, 0, t, t[4:], t[8:], wf, lay, 1, zs.AdamWHParams())
    torch.cuda.synchronize()
    assert bool((wf == 3.0).all())


# ---------------------------------------------------------------------------
# reduce + accumulate + gated AdamW (the stage-2 accumulation path)


def _accum_case(n_dp, length, micro, inject=None, cfg=100, wdt=zs.ZERO_BF16):
    """micro-batches of fp16 rows reduced into acc, then AdamW gated on the
    overflow flag; inject = (micro-batch, row, index, bits) plants a
    non-finite gradient."""
    draw = GradDraw(F16, 1e-3, scale=65536.0)
    lay, _ = zs.zero_flatten_layout([length * n_dp], n_dp, 8)
    s = lay.shard
    rank = 1 % n_dp
    lo = rank * s
    scale = 1.0 / (n_dp * 65536.0 * micro)
    w = host_master(cfg, lo, s)
    m = np.zeros(s, np.float32)
    v = np.zeros(s, np.float32)
    acc = np.zeros(s, np.float32)
    wout = np.full(lay.n_pad, CANARY, np.uint16)
    dw, dm, dv, dacc = devf(w), devf(m), devf(v), devf(acc)
    dwf = dev16(wout, wdt)
    d_ovf = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_ss = torch.zeros(1, dtype=torch.float64, device="cuda")
    o_ovf = np.zeros(1, np.uint32)
    o_ss = np.zeros(1, np.float64)
    for mb in range(micro):
        rows = host_rows(cfg, 1, mb, n_dp, lo, s, draw)
        if inject is not None and inject[0] == mb:
            rows[inject[1], inject[2]] = inject[3]
        zs.zero_shard_reduce(dev16(rows, zs.ZERO_FP16), n_dp, s, s, dacc, accumulate=mb > 0,
                             overflow=d_ovf, sumsq=d_ss if mb == micro - 1 else None)
        oracle.reduce(rows, oracle.FP16, n_dp, s, s, acc, mb > 0, overflow=o_ovf,
                      sumsq=o_ss if mb == micro - 1 else None)
    hp = zs.AdamWHParams(step=1, grad_scale=scale, **HP)
    zs.zero_shard_adamw(dacc, dw, dm, dv, dwf, lay, rank, hp, skip=d_ovf)
    slot = wout[lo:lo + s].copy()
    oracle.adamw(acc, w, m, v, slot, wdt, s, 1, grad_scale=scale, skip=o_ovf, **HP)
    wout[lo:lo + s] = slot
    torch.cuda.synchronize()
    assert int(d_ovf.item()) == int(o_ovf[0])
    diff = check_f32(hostf(dacc), acc, "acc")
    diff += check_f32(hostf(dw), w, "master") + check_f32(hostf(dm), m, "m")
    diff += check_f32(hostf(dv), v, "v") + check_16(host16(dwf), wout, wdt, "weights")
    assert diff == 0
    ref = float(o_ss[0])
    if np.isfinite(ref):
        assert abs(d_ss.item() - ref) <= 1e-10 * ref
    return int(o_ovf[0])


@pytest.mark.parametrize("n_dp,micro", [(8, 4), (3, 2), (1, 1)])
def test_accumulate_then_adamw(n_dp, micro):
    assert _accum_case(n_dp, 40_000 + 3, micro) == 0


@pytest.mark.parametrize("where", ["first", "middle", "last"])
@pytest.mark.parametrize("mb", [0, 3])
@pytest.mark.parametrize("bits", [0x7C00, 0xFE00])
def test_overflow_skips_the_step(where, mb, bits):
    length = 40_000
    s = length  # shard of a [length * 8] vector over 8 ranks with align 8
    idx = {"first": 0, "middle": s // 2 + 3, "last": s - 1}[where]
    assert _accum_case(8, length, 4, inject=(mb, 5, idx, bits), cfg=101) == 1


@pytest.mark.parametrize("plant,idx", [
    ({2: 0x7F80}, 1234),                 # +Inf
    ({0: 0xFF80}, 4095),                 # -Inf at the last element (the tail of the launch)
    ({3: 0x7FC1}, 7),                    # a NaN
    ({1: 0x7F80, 2: 0xFF80}, 2048),      # +Inf + -Inf: NaN from finite-looking rows
])
def test_overflow_flag_of_fused_step_and_update_applied(plant, idx):
    """The fused step reports a non-finite reduced gradient (and, being one
    pass, still applies the update, like the oracle): Inf and NaN propagate
    through m, v, the master and the cast exactly as in the oracle."""
    draw = GradDraw(BF16, 1e-3)
    n_dp, s = 4, 4096 + 3                # a 3-element tail after the quads
    lay, _ = zs.zero_flatten_layout([n_dp * s], n_dp)
    rows = host_rows(102, 1, 0, n_dp, s, s, draw)
    for k, bits in plant.items():
        rows[k, idx] = bits
    w = host_master(102, s, s)
    m = np.zeros(s, np.float32)
    v = np.zeros(s, np.float32)
    wout = np.zeros(lay.n_pad, np.uint16)
    dw, dm, dv, dwf = devf(w), devf(m), devf(v), dev16(wout, 0)
    d_ovf = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_shard_step(dev16(rows, 0), s, s, dw, dm, dv, dwf, lay, 1,
                       zs.AdamWHParams(step=1, grad_scale=0.25, **HP), overflow=d_ovf)
    o_ovf = np.zeros(1, np.uint32)
    slot = wout[s:2 * s].copy()
    oracle.step(rows, 0, n_dp, s, s, w, m, v, slot, 0, 1, grad_scale=0.25, overflow=o_ovf, **HP)
    torch.cuda.synchronize()
    assert int(d_ovf.item()) == 1 == int(o_ovf[0])
    assert check_f32(hostf(dw), w, "master") + check_16(host16(dwf)[s:2 * s], slot, 0, "w") == 0
    assert check_f32(hostf(dm), m, "m") + check_f32(hostf(dv), v, "v") == 0
    assert not np.isfinite(w[idx]) and np.all(np.isfinite(np.delete(w, idx)))


# ---------------------------------------------------------------------------
# the cast, exhaustively: AdamW with lr = 0 and a zero gradient leaves every
# fp32 pattern unchanged, so the slot receives the 16-bit cast of every pattern


@pytest.mark.parametrize("wdt", [zs.ZERO_BF16, zs.ZERO_FP16])
def test_cast_every_fp32_pattern(wdt):
    chunk = 1 << 28
    lay, _ = zs.zero_flatten_layout([chunk], 1, 8)
    dev = torch.device("cuda")
    acc = torch.zeros(chunk, dtype=torch.float32, device=dev)
    dm = torch.zeros(chunk, dtype=torch.float32, device=dev)
    dv = torch.zeros(chunk, dtype=torch.float32, device=dev)
    out = torch.empty(chunk, dtype=zs_tdt(wdt), device=dev)
    base = torch.arange(chunk, dtype=torch.int64, device=dev)
    hbase = np.arange(chunk, dtype=np.uint32)
    hp = zs.AdamWHParams(lr=0.0, weight_decay=0.0, step=1)
    for c in range(0, 1 << 32, chunk):
        pat = base + c  # fp32 bit patterns [c, c + chunk) as int32
        dw = torch.where(pat >= (1 << 31), pat - (1 << 32), pat).to(torch.int32).view(torch.float32)
        dm.zero_()
        dv.zero_()
        zs.zero_shard_adamw(acc, dw, dm, dv, out, lay, 0, hp)
        got = host16(out)
        x = (hbase + np.uint32(c)).view(np.float32)
        ref = oracle.f32_to_bf16(x) if wdt == zs.ZERO_BF16 else oracle.f32_to_f16(x)
        bad = got != ref
        if bad.any():  # only NaN payloads may differ
            from tests.gpu_util import is_nan16
            assert np.all(is_nan16(got[bad], wdt) & is_nan16(ref[bad], wdt)), \
                f"cast mismatch at fp32 pattern {x.view(np.uint32)[bad][0]:#x}"


def zs_tdt(dt):
    return torch.bfloat16 if dt == zs.ZERO_BF16 else torch.float16


@pytest.mark.parametrize("n_dp,length,lead", [(3, 1_048_589, 0), (8, 300_001, 0), (8, 70_001, 1)])
def test_sum_of_squares_is_reproducible(n_dp, length, lead):
    """The sum of squares goes through per-workgroup partials and a fixed-
    order finish: the same inputs give the same bits on every call (the
    quad kernel with a ragged tail, or -- lead 1, unaligned rows -- the
    element kernel alone), for the fused step and the reduce; and the value
    is the oracle's sequential fp64 sum of g^2 within 1e-10 relative (the
    summation orders differ; n * 2^-53 bounds the sequential sum's error
    for 10^6 positive terms)."""
    draw = GradDraw(BF16, 1e-3)
    rows = host_rows(150 + n_dp, 1, 0, n_dp, 0, length, draw)
    lay, _ = zs.zero_flatten_layout([length * n_dp], n_dp)
    buf = np.zeros(n_dp * length + lead, np.uint16)
    buf[lead:] = rows.reshape(-1)
    g = dev16(buf, zs.ZERO_BF16)[lead:]
    w0 = host_master(150 + n_dp, 0, length)
    hp = zs.AdamWHParams(step=1, grad_scale=1.0 / n_dp, **HP)
    sums = []
    for _ in range(2):
        dw, dm, dv = devf(w0), devf(np.zeros(length, np.float32)), devf(np.zeros(length, np.float32))
        wf = torch.zeros(lay.n_pad, dtype=torch.bfloat16, device="cuda")
        ss = torch.zeros(1, dtype=torch.float64, device="cuda")
        zs.zero_shard_step(g, length, length, dw, dm, dv, wf, lay, 0, hp, sumsq=ss)
        acc = torch.empty(length, device="cuda")
        rs = torch.zeros(1, dtype=torch.float64, device="cuda")
        zs.zero_shard_reduce(g, n_dp, length, length, acc, sumsq=rs)
        torch.cuda.synchronize()
        sums.append((ss.item(), rs.item()))
    assert np.array(sums[0]).view(np.uint64).tolist() == np.array(sums[1]).view(np.uint64).tolist()
    o_ss = np.zeros(1)
    w, m, v = w0.copy(), np.zeros(length, np.float32), np.zeros(length, np.float32)
    oracle.step(rows, oracle.BF16, n_dp, length, length, w, m, v, np.zeros(length, np.uint16),
                oracle.BF16, 1, grad_scale=1.0 / n_dp, sumsq=o_ss, **HP)
    o_rs = np.zeros(1)
    oracle.reduce(rows, oracle.BF16, n_dp, length, length, np.zeros(length, np.float32), False,
                  sumsq=o_rs)
    assert abs(sums[0][0] - o_ss[0]) <= 1e-10 * o_ss[0]
    assert abs(sums[0][1] - o_rs[0]) <= 1e-10 * o_rs[0]


@pytest.mark.parametrize("wdt", [zs.ZERO_BF16, zs.ZERO_FP16])
def test_subnormal_operands_are_kept(wdt):
    """No flush to zero on either side: bf16 gradient rows half of them
    subnormal, and master, m, v mixing subnormal and small normal binary32
    values; an inexact gradient scale (1/3) makes products land in the
    subnormal range too.  Fused step (vector path and tail) and reduce,
    bitwise against the oracle."""
    rng = np.random.default_rng(77)
    n_dp, n = 3, 100_003
    lay, _ = zs.zero_flatten_layout([n * n_dp], n_dp)

    def bf16_mix(size):
        h = rng.integers(0, 1 << 7, size=size).astype(np.uint16)         # subnormal bf16
        normal = rng.random(size) < 0.5
        h[normal] = (rng.integers(1, 20, size=int(normal.sum())) << 7 |
                     rng.integers(0, 1 << 7, size=int(normal.sum()))).astype(np.uint16)
        return h | (rng.integers(0, 2, size=size).astype(np.uint16) << 15)

    def f32_mix(size, positive=False):
        mant = rng.integers(1, 1 << 23, size=size).astype(np.uint32)
        exp = np.where(rng.random(size) < 0.5, 0, rng.integers(1, 12, size=size)).astype(np.uint32)
        sign = np.zeros(size, np.uint32) if positive else \
            rng.integers(0, 2, size=size).astype(np.uint32) << 31
        return (sign | exp << 23 | mant).view(np.float32)

    rows = np.stack([bf16_mix(n) for _ in range(n_dp)])
    w, m, v = f32_mix(n), f32_mix(n), f32_mix(n, positive=True)
    assert np.count_nonzero((w.view(np.uint32) & 0x7F800000) == 0) > n // 4
    dw, dm, dv = devf(w), devf(m), devf(v)
    dwf = dev16(np.zeros(lay.n_pad, np.uint16), wdt)
    g = dev16(rows, zs.ZERO_BF16)
    hp = zs.AdamWHParams(step=2, grad_scale=1.0 / 3.0, **HP)
    zs.zero_shard_step(g, n, n, dw, dm, dv, dwf, lay, 0, hp)
    slot = np.zeros(n, np.uint16)
    oracle.step(rows, oracle.BF16, n_dp, n, n, w, m, v, slot, wdt, 2, grad_scale=1.0 / 3.0, **HP)
    torch.cuda.synchronize()
    diff = check_f32(hostf(dw), w, "master") + check_f32(hostf(dm), m, "m")
    diff += check_f32(hostf(dv), v, "v") + check_16(host16(dwf)[:n], slot, wdt, "weights")
    assert diff == 0
    acc = torch.empty(n, device="cuda")
    zs.zero_shard_reduce(g, n_dp, n, n, acc)
    o_acc = np.zeros(n, np.float32)
    oracle.reduce(rows, oracle.BF16, n_dp, n, n, o_acc, False)
    torch.cuda.synchronize()
    assert check_f32(hostf(acc), o_acc, "acc") == 0
    assert np.count_nonzero((o_acc.view(np.uint32) & 0x7F800000) == 0) > n // 20
