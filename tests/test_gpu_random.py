"""Seeded random cases of the fused step, the reduce, the 8-bit step and
AdamW (with and without its controls) against the oracle,
bitwise: row count, range length, row stride, rank, shard offset, gradient
and weight formats, the flags, and -- by leading elements before each
buffer -- the alignment of every pointer, so that calls mix the vector
kernels, their ragged tails and the element kernels in ways the
hand-picked cases do not.  The arithmetic is the sharded step of "ZeRO and
FSDP" (A sharded Adam step); the bar is the same as everywhere: every
element bit-identical, the sum of squares within its bound."""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_flatten_amd as zs
from synth import BF16, F16, F32
from synth.synth_const import BUF_GRAD
from synth.workloads import GradDraw
from tests.gpu_util import check_16, check_f32, host_master, host_rows

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
ODT = {BF16: oracle.BF16, F16: oracle.FP16, F32: oracle.FP32}
TDT = {zs.ZERO_BF16: torch.bfloat16, zs.ZERO_FP16: torch.float16}
CANARY = 0x5A5A


def _lead(a: np.ndarray, lead: int, tdt=None):
    """Device copy of host array a starting `lead` elements into a fresh
    buffer (so the pointer is off 16-byte alignment by lead * itemsize)."""
    if a.dtype == np.uint16:
        buf = np.zeros(a.size + lead, np.uint16)
        buf[lead:] = a.reshape(-1)
        return torch.from_numpy(buf.view(np.int16)).cuda().view(tdt)[lead:]
    buf = np.zeros(a.size + lead, a.dtype)
    buf[lead:] = a.reshape(-1)
    return torch.from_numpy(buf).cuda()[lead:]


def _host(t):
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


def _case(seed):
    r = np.random.default_rng(seed)
    n_dp = int(r.choice([1, 2, 3, 5, 8, 13, 64]))
    shard = int(r.integers(1, 40_000 if n_dp == 64 else 200_000))
    off = int(r.integers(0, shard)) if r.random() < 0.5 else 0
    length = int(r.integers(0, shard - off + 1)) if r.random() < 0.3 else shard - off
    pad = int(r.choice([0, 0, 4, 7, 64]))
    kind = [BF16, F16, F32][int(r.integers(0, 3))]
    wdt = [zs.ZERO_BF16, zs.ZERO_FP16][int(r.integers(0, 2))]
    leads = [int(r.choice([0, 0, 1, 2, 3])) for _ in range(5)]   # grads, master, m, v, sums
    return dict(n_dp=n_dp, shard=shard, off=off, length=length, ld=length + pad, kind=kind,
                wdt=wdt, leads=leads, rank=int(r.integers(0, n_dp)),
                ovf=bool(r.random() < 0.5), ssq=bool(r.random() < 0.5))


@pytest.mark.parametrize("seed", range(12))
def test_random_step(seed):
    c = _case(1000 + seed)
    print(f"\n[random step] {c}", flush=True)
    n_dp, S, off, L, ld = c["n_dp"], c["shard"], c["off"], c["length"], c["ld"]
    lay, _ = zs.zero_flatten_layout([S * n_dp], n_dp)
    assert lay.shard == S
    draw = GradDraw(c["kind"], 1e-3, outlier_p=0.01, outlier_mul=100.0)
    lo = c["rank"] * S + off
    w = host_master(200 + seed, lo, L)
    m = np.zeros(L, np.float32)
    v = np.zeros(L, np.float32)
    wout = np.full(lay.n_pad, CANARY, np.uint16)
    g_lead, w_lead, m_lead, v_lead, _ = c["leads"]
    dw, dm, dv = _lead(w, w_lead), _lead(m, m_lead), _lead(v, v_lead)
    dwf = torch.from_numpy(wout.view(np.int16).copy()).cuda().view(TDT[c["wdt"]])
    for t in (1, 2):
        rows = host_rows(200 + seed, t, 0, n_dp, lo, L, draw) if L > 0 else \
            np.zeros((n_dp, 0), np.float32 if c["kind"] == F32 else np.uint16)
        slab = np.zeros((n_dp, ld), rows.dtype)
        slab[:, :L] = rows
        g = _lead(slab, g_lead, torch.bfloat16 if c["kind"] == BF16 else torch.float16)
        hp = zs.AdamWHParams(step=t, grad_scale=1.0 / n_dp, **HP)
        d_ovf = torch.zeros(1, dtype=torch.int32, device="cuda") if c["ovf"] else None
        d_ss = torch.zeros(1, dtype=torch.float64, device="cuda") if c["ssq"] else None
        if seed % 2:  # odd seeds: the constants from a device buffer
            consts = zs.new_step_consts()
            consts.copy_(torch.from_numpy(zs.zero_step_consts_make(hp)))
            zs.zero_shard_step_dc(g, ld, L, dw, dm, dv, dwf, lay, c["rank"], consts,
                                  shard_off=off, overflow=d_ovf, sumsq=d_ss)
        else:
            zs.zero_shard_step(g, ld, L, dw, dm, dv, dwf, lay, c["rank"], hp, shard_off=off,
                               overflow=d_ovf, sumsq=d_ss)
        o_ovf, o_ss = np.zeros(1, np.uint32), np.zeros(1)
        slot = wout[lo:lo + L].copy()
        if L > 0:
            oracle.step(np.ascontiguousarray(slab.reshape(-1)), ODT[c["kind"]], n_dp, ld, L, w, m,
                        v, slot, c["wdt"], t, grad_scale=1.0 / n_dp, overflow=o_ovf, sumsq=o_ss,
                        **HP)
        wout[lo:lo + L] = slot
        torch.cuda.synchronize()
        diff = check_f32(_host(dw), w, "master") + check_f32(_host(dm), m, "m")
        diff += check_f32(_host(dv), v, "v")
        got = _host(dwf)
        diff += check_16(got[lo:lo + L], wout[lo:lo + L], c["wdt"], "weights")
        assert diff == 0
        assert np.array_equal(got[:lo], wout[:lo]) and np.array_equal(got[lo + L:], wout[lo + L:])
        if c["ovf"]:
            assert int(d_ovf.item()) == int(o_ovf[0])
        if c["ssq"]:
            assert abs(d_ss.item() - o_ss[0]) <= 1e-10 * o_ss[0]


@pytest.mark.parametrize("seed", range(10))
def test_random_reduce(seed):
    c = _case(2000 + seed)
    n_dp, L, ld = c["n_dp"], c["length"], c["ld"]
    acc_mode = seed % 2 == 1
    print(f"\n[random reduce] {c} accumulate={acc_mode}", flush=True)
    draw = GradDraw(c["kind"], 1e-3)
    rows = host_rows(220 + seed, 1, 0, n_dp, 0, L, draw) if L > 0 else \
        np.zeros((n_dp, 0), np.float32 if c["kind"] == F32 else np.uint16)
    slab = np.zeros((n_dp, ld), rows.dtype)
    slab[:, :L] = rows
    g = _lead(slab, c["leads"][0], torch.bfloat16 if c["kind"] == BF16 else torch.float16)
    acc = host_master(240 + seed, 0, L, sigma=1e-3) if acc_mode else np.zeros(L, np.float32)
    dacc = _lead(acc, c["leads"][1])
    d_ovf = torch.zeros(1, dtype=torch.int32, device="cuda") if c["ovf"] else None
    d_ss = torch.zeros(1, dtype=torch.float64, device="cuda") if c["ssq"] else None
    zs.zero_shard_reduce(g, n_dp, ld, L, dacc, accumulate=acc_mode, overflow=d_ovf, sumsq=d_ss)
    o_ovf, o_ss = np.zeros(1, np.uint32), np.zeros(1)
    if L > 0:
        oracle.reduce(np.ascontiguousarray(slab.reshape(-1)), ODT[c["kind"]], n_dp, ld, L, acc,
                      acc_mode, overflow=o_ovf, sumsq=o_ss)
    torch.cuda.synchronize()
    assert check_f32(_host(dacc), acc, "acc") == 0
    if c["ovf"]:
        assert int(d_ovf.item()) == int(o_ovf[0])
    if c["ssq"] and L > 0:
        assert abs(d_ss.item() - o_ss[0]) <= 1e-10 * o_ss[0]


@pytest.mark.parametrize("seed", range(8))
def test_random_q8_step(seed):
    """The fused 8-bit step within its stated requirements (shard and shard
    offset multiples of 256, code rows 4-byte aligned, state 16-byte
    aligned), everything else random: row count, range length and partial
    last block, row and scale strides, rank, flags; codes from the oracle's
    quantizer."""
    r = np.random.default_rng(3000 + seed)
    B = zs.ZERO_Q8_BLOCK
    n_dp = int(r.choice([1, 2, 3, 8, 13, 64]))
    S = B * int(r.integers(1, 60 if n_dp == 64 else 600))
    off = B * int(r.integers(0, S // B)) if r.random() < 0.5 else 0
    L = int(r.integers(1, S - off + 1)) if r.random() < 0.5 else S - off
    ld = (L + 3) // 4 * 4 + 4 * int(r.integers(0, 20))   # a multiple of 4 (required)
    nb = zs.q8_blocks(L)
    sld = nb + int(r.integers(0, 5))
    rank = int(r.integers(0, n_dp))
    ovf, ssq = bool(r.random() < 0.5), bool(r.random() < 0.5)
    q_lead = 4 * int(r.integers(0, 3))
    print(f"\n[random q8] n_dp={n_dp} S={S} off={off} L={L} ld={ld} sld={sld} rank={rank} "
          f"ovf={ovf} ssq={ssq} lead={q_lead}", flush=True)
    lay, _ = zs.zero_flatten_layout([S * n_dp], n_dp, B)
    assert lay.shard == S
    gq = np.zeros((n_dp, ld), np.int8)
    gs = np.zeros((n_dp, sld), np.float32)
    for k in range(n_dp):
        x = synth.fill_host(F32, 0, synth.tag(BUF_GRAD, 250, seed, 0, k), 0, L, 1e-3)
        q, s = oracle.q8_quantize(x, oracle.FP32)
        gq[k, :L], gs[k, :nb] = q, s
    lo = rank * S + off
    w = host_master(250, lo, L)
    m, v = np.zeros(L, np.float32), np.zeros(L, np.float32)
    o_wq = np.full(lay.n_pad, 0x33, np.int8)
    o_ws = np.full(lay.n_pad // B, -3.0, np.float32)
    dgq = _lead(gq, q_lead)
    dgs = torch.from_numpy(gs.reshape(-1).copy()).cuda()
    dw, dm, dv = (torch.from_numpy(a.copy()).cuda() for a in (w, m, v))
    dwq = torch.from_numpy(o_wq.copy()).cuda()
    dws = torch.from_numpy(o_ws.copy()).cuda()
    d_ovf = torch.zeros(1, dtype=torch.int32, device="cuda") if ovf else None
    d_ss = torch.zeros(1, dtype=torch.float64, device="cuda") if ssq else None
    hp = zs.AdamWHParams(step=1, grad_scale=1.0 / n_dp, **HP)
    zs.zero_shard_step_q8(dgq, dgs, ld, sld, L, dw, dm, dv, dwq, dws, lay, rank, hp,
                          shard_off=off, overflow=d_ovf, sumsq=d_ss)
    o_ovf, o_ss = np.zeros(1, np.uint32), np.zeros(1)
    s_wq = o_wq[lo:lo + L].copy()
    s_ws = o_ws[lo // B:lo // B + nb].copy()
    oracle.step_q8(gq.reshape(-1), gs.reshape(-1), n_dp, ld, sld, L, w, m, v, s_wq, s_ws, 1,
                   grad_scale=1.0 / n_dp, overflow=o_ovf, sumsq=o_ss, **HP)
    o_wq[lo:lo + L] = s_wq
    o_ws[lo // B:lo // B + nb] = s_ws
    torch.cuda.synchronize()
    assert check_f32(_host(dw), w, "master") + check_f32(_host(dm), m, "m") + \
        check_f32(_host(dv), v, "v") == 0
    assert np.array_equal(dwq.cpu().numpy(), o_wq)
    assert np.array_equal(dws.cpu().numpy().view(np.uint32), o_ws.view(np.uint32))
    if ovf:
        assert int(d_ovf.item()) == int(o_ovf[0])
    if ssq:
        assert abs(d_ss.item() - o_ss[0]) <= 1e-10 * o_ss[0]


@pytest.mark.parametrize("seed", range(10))
def test_random_adamw(seed):
    """AdamW from an fp32 gradient buffer -- the plain entry point, or the
    one with controls in any mix (skip flag, clipping from a sum of squares
    to a random norm, a device loss scale) -- on random ranges, shard
    offsets and pointer alignments, non-zero moments, two steps, bitwise
    against the oracle, canaries around the slot."""
    c = _case(4000 + seed)
    n_dp, S, off, L = c["n_dp"], c["shard"], c["off"], c["length"]
    lay, _ = zs.zero_flatten_layout([S * n_dp], n_dp)
    lo = c["rank"] * S + off
    # the controls cycle with the seed so that each runs un-skipped: clipping
    # that bites (seeds 1, 5; with a loss scale on 1), a loss scale alone (4),
    # a sum too small to clip (7), controls all absent (8), a skipped step (2)
    ex = seed % 3 != 0
    skip_v = (None, 0, 1, 0)[seed % 4]
    scale = (None, 1024.0, 65536.0)[(seed + 1) % 3] if ex else None
    base = (None, 1e6, 1e2, 1e-6)[seed % 4] if ex else None
    ssq_v = base * (scale or 1.0) ** 2 if base is not None else None
    max_norm = (0.5, 1.0)[seed % 2] if ssq_v is not None else 0.0
    print(f"\n[random adamw] {c} ex={ex} skip={skip_v} sumsq={ssq_v} max_norm={max_norm} "
          f"loss_scale={scale}", flush=True)
    gs = 1.0 / n_dp
    if ssq_v is not None:
        s = float(np.float32(gs / scale)) if scale else float(np.float32(gs))
        bites = oracle.clip_coef(ssq_v, s, max_norm) < 1.0
        assert bites if seed in (1, 5) else (not bites if seed == 7 else True)
    acc = host_master(150 + seed, lo, L, sigma=1e-3 * (scale or 1.0))
    w = host_master(160 + seed, lo, L)
    m = host_master(170 + seed, lo, L, sigma=1e-4)
    v = np.abs(host_master(180 + seed, lo, L, sigma=1e-8))
    wout = np.full(lay.n_pad, CANARY, np.uint16)
    leads = c["leads"]
    dacc, dw, dm, dv = (_lead(a, k) for a, k in zip((acc, w, m, v), leads))
    dwf = torch.from_numpy(wout.view(np.int16).copy()).cuda().view(TDT[c["wdt"]])
    d_skip = (torch.tensor([skip_v], dtype=torch.int32, device="cuda")
              if skip_v is not None else None)
    d_ss = torch.tensor([ssq_v], dtype=torch.float64, device="cuda") if ssq_v is not None else None
    d_ls = zs.new_loss_scale(scale) if scale is not None else None
    o_skip = np.array([skip_v], np.uint32) if skip_v is not None else None
    o_ss = np.array([ssq_v]) if ssq_v is not None else None
    o_ls = np.array([scale], np.float32) if scale is not None else None
    for t in (1, 2):
        hp = zs.AdamWHParams(step=t, grad_scale=gs, **HP)
        if ex and seed % 2:  # odd seeds: the constants from a device buffer
            consts = zs.new_step_consts()
            consts.copy_(torch.from_numpy(zs.zero_step_consts_make(hp)))
            zs.zero_shard_adamw_dc(dacc, dw, dm, dv, dwf, lay, c["rank"], consts, shard_off=off,
                                   length=L, skip=d_skip, sumsq=d_ss, max_norm=max_norm,
                                   loss_scale=d_ls)
        elif ex:
            zs.zero_shard_adamw_ex(dacc, dw, dm, dv, dwf, lay, c["rank"], hp, shard_off=off,
                                   length=L, skip=d_skip, sumsq=d_ss, max_norm=max_norm,
                                   loss_scale=d_ls)
        else:
            zs.zero_shard_adamw(dacc, dw, dm, dv, dwf, lay, c["rank"], hp, shard_off=off,
                                length=L, skip=d_skip)
        slot = wout[lo:lo + L].copy()
        if L > 0:
            if ex:
                oracle.adamw_ex(acc, w, m, v, slot, c["wdt"], L, t, grad_scale=gs, skip=o_skip,
                                sumsq=o_ss, max_norm=max_norm, loss_scale=o_ls, **HP)
            else:
                oracle.adamw(acc, w, m, v, slot, c["wdt"], L, t, grad_scale=gs, skip=o_skip, **HP)
        wout[lo:lo + L] = slot
        torch.cuda.synchronize()
        diff = check_f32(_host(dw), w, "master") + check_f32(_host(dm), m, "m")
        diff += check_f32(_host(dv), v, "v")
        got = _host(dwf)
        diff += check_16(got[lo:lo + L], wout[lo:lo + L], c["wdt"], "weights")
        assert diff == 0
        assert np.array_equal(got[:lo], wout[:lo]) and np.array_equal(got[lo + L:], wout[lo + L:])
        assert np.array_equal(_host(dacc), acc)
