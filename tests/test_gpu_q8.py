"""GPU parity (through the C ABI) of the 8-bit blockwise communication path
(ZeRO++'s quantized weight all-gather and gradient reduce-scatter, "ZeRO and
FSDP", FSDP section; "ZeRO Optimizer, in depth", "Offload and ZeRO++")
against the oracle, bit for bit: the quantizer, the dequantizer, and the
fused step that reads 8-bit rows and writes 8-bit weights.  The quantizer
itself is this library's reading (the pages give none): parity with the
pages is unpinned, parity with the oracle is exact."""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_flatten_amd as zs
from synth import BF16, F16, F32, tag
from synth.synth_const import BUF_GRAD, BUF_MASTER, outlier_threshold
from synth.workloads import workload
from tests.gpu_util import check_16

pytestmark = pytest.mark.gpu

B = zs.ZERO_Q8_BLOCK
HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
ODT = {F32: oracle.FP32, BF16: oracle.BF16, F16: oracle.FP16}
TDT = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}


def _draw(kind, n, seed, cfg=160, sigma=1.0):
    return synth.fill_host(kind, seed, tag(BUF_GRAD, cfg, 0, 0, seed), 0, n, sigma,
                           outlier_threshold(0.01), 100.0)


def _dev(a, kind):
    t = torch.from_numpy(a.copy())
    if kind != F32:
        t = t.view(torch.int16).view(TDT[kind])
    return t.cuda()


def _same_f32(a, b):
    """bitwise, NaN matching NaN"""
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32))


@pytest.mark.parametrize("kind", [F32, BF16, F16])
@pytest.mark.parametrize("n,lead", [(1, 0), (255, 0), (256, 0), (257, 1), (100_003, 0),
                                    (1_048_589, 3), (513, 8), (100_003, 8)])
def test_quantize_and_dequantize_bitwise(kind, n, lead):
    x = _draw(kind, n, n % 97 + lead)
    if n > 3 * B:  # a zero block, an infinite block, a NaN block
        inf = np.float32(np.inf) if kind == F32 else np.uint16(0x7F80 if kind == BF16 else 0x7C00)
        nan = np.float32(np.nan) if kind == F32 else np.uint16(0x7FC0 if kind == BF16 else 0x7E00)
        x[:B] = 0
        x[B + 3] = inf
        x[2 * B + 7] = nan
    d = _dev(np.concatenate([np.zeros(lead, x.dtype), x]), kind)[lead:]
    q = torch.empty(n + lead, dtype=torch.int8, device="cuda")[lead:]
    # the scales off 16-byte alignment too when lead > 0 (the quantizer then
    # stores them one by one); lead 8 keeps the codes 8-byte and 16-bit
    # values 16-byte aligned (the vector path of the 16-bit dequantize) at an
    # offset
    s = torch.empty(zs.q8_blocks(n) + lead, dtype=torch.float32, device="cuda")[lead:]
    zs.zero_q8_quantize(d, q, s)
    oq, os_ = oracle.q8_quantize(x, ODT[kind])
    assert np.array_equal(q.cpu().numpy(), oq)
    assert _same_f32(s.cpu().numpy(), os_)
    for ydt in (F32, BF16, F16):
        y = torch.empty(n + lead, dtype=TDT[ydt], device="cuda")[lead:]
        zs.zero_q8_dequantize(q, s, y)
        oy = oracle.q8_dequantize(oq, os_, ODT[ydt])
        got = y.cpu()
        got = got.numpy() if ydt == F32 else got.view(torch.int16).numpy().view(np.uint16)
        if ydt == F32:
            assert _same_f32(got, oy)
        else:  # NaN positions equal (their sign and payload are the platform's), the rest bitwise
            assert check_16(got, oy, ODT[ydt], "dequantized") == 0


def _q8_rows(n_dp, ld, seed, cfg, t=1):
    """n_dp rows of ld fp32 draws, quantized by the oracle: codes [n_dp][ld],
    scales [n_dp][ld / B]."""
    qs, ss = [], []
    for k in range(n_dp):
        x = synth.fill_host(F32, seed, tag(BUF_GRAD, cfg, t, 0, k), 0, ld, 1e-3,
                            outlier_threshold(0.01), 100.0)
        q, s = oracle.q8_quantize(x, oracle.FP32)
        qs.append(q)
        ss.append(s)
    return np.stack(qs), np.stack(ss)


@pytest.mark.parametrize("n_dp", [1, 3, 8, 64])
@pytest.mark.parametrize("ragged", [False, True])
@pytest.mark.parametrize("dc", [False, True])
def test_fused_q8_step_bitwise(n_dp, ragged, dc):
    """dc: the constants from a device buffer (zero_shard_step_q8_dc),
    written before each step -- the same results bit for bit."""
    shard = 64 * B if n_dp <= 8 else 16 * B
    lay, _ = zs.zero_flatten_layout([shard * n_dp], n_dp, B)
    S = lay.shard
    rank = n_dp - 1
    length = S - 77 if ragged else S
    ld = S + 4 * B  # rows wider than the range
    sld = ld // B
    w = synth.fill_host(F32, 0, tag(BUF_MASTER, 161), 0, length, 0.02)
    m, v = np.zeros(length, np.float32), np.zeros(length, np.float32)
    dw, dm, dv = (torch.from_numpy(a.copy()).cuda() for a in (w, m, v))
    CAN = 0x5A
    wq = torch.full((lay.n_pad,), CAN, dtype=torch.int8, device="cuda")
    wsc = torch.full((lay.n_pad // B,), -7.0, device="cuda")
    o_wq = np.zeros(length, np.int8)
    o_ws = np.zeros(zs.q8_blocks(length), np.float32)
    for t in (1, 2, 3):
        gq, gs = _q8_rows(n_dp, ld, 1, 162 + n_dp, t)
        if t == 2:  # a NaN block in one row: the whole block reads as NaN, the flag rises
            gs[n_dp // 2, 1] = np.nan
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        ss = torch.zeros(1, dtype=torch.float64, device="cuda")
        hp = zs.AdamWHParams(step=t, grad_scale=1.0 / n_dp, **HP)
        dgq, dgs = torch.from_numpy(gq.reshape(-1)).cuda(), torch.from_numpy(gs.reshape(-1)).cuda()
        if dc:
            consts = zs.new_step_consts()
            consts.copy_(torch.from_numpy(zs.zero_step_consts_make(hp)))
            zs.zero_shard_step_q8_dc(dgq, dgs, ld, sld, length, dw, dm, dv, wq, wsc, lay, rank,
                                     consts, overflow=flag, sumsq=ss)
        else:
            zs.zero_shard_step_q8(dgq, dgs, ld, sld, length, dw, dm, dv, wq, wsc, lay, rank, hp,
                                  overflow=flag, sumsq=ss)
        o_flag = np.zeros(1, np.uint32)
        o_ss = np.zeros(1)
        oracle.step_q8(gq.reshape(-1), gs.reshape(-1), n_dp, ld, sld, length, w, m, v, o_wq, o_ws,
                       t, grad_scale=1.0 / n_dp, overflow=o_flag, sumsq=o_ss, **HP)
        torch.cuda.synchronize()
        assert int(flag.item()) == int(o_flag[0]) == (1 if t == 2 else 0)
        if t != 2:
            assert abs(ss.item() - o_ss[0]) <= 1e-9 * o_ss[0]
        assert _same_f32(dw.cpu().numpy(), w) and _same_f32(dm.cpu().numpy(), m)
        assert _same_f32(dv.cpu().numpy(), v)
        lo = rank * S
        got_q = wq.cpu().numpy()
        assert np.array_equal(got_q[lo:lo + length], o_wq)
        assert np.all(got_q[:lo] == CAN) and np.all(got_q[lo + length:] == CAN)
        got_s = wsc.cpu().numpy()
        nb = zs.q8_blocks(length)
        assert _same_f32(got_s[lo // B:lo // B + nb], o_ws)
        assert np.all(got_s[:lo // B] == -7.0) and np.all(got_s[lo // B + nb:] == -7.0)


def test_q8_step_full_size_sampled_blocks():
    """The 7B list over 8 ranks, rank 1 (842,301,952 elements = 3,290,242
    blocks), int8 rows quantized on the device from fp32 draws, t = 1, 2:
    the device quantizer and the step checked against the oracle on 200
    whole sampled blocks (a block's codes depend on all of its elements)."""
    wl = workload(6)
    lay, _ = zs.zero_flatten_layout(wl.numels, wl.n_dp, B)
    S, n_dp, rank = lay.shard, wl.n_dp, wl.rank
    print(f"\n[full] q8 step S={S} n_dp={n_dp} rank={rank}", flush=True)
    nb = S // B
    d = wl.grad
    rows_q = torch.empty((n_dp, S), dtype=torch.int8, device="cuda")
    rows_s = torch.empty((n_dp, nb), dtype=torch.float32, device="cuda")
    tmp = torch.empty(S, dtype=torch.float32, device="cuda")
    W = torch.empty(S, device="cuda")
    synth.fill_device(W, F32, wl.seed, tag(BUF_MASTER, wl.cid), rank * S, wl.master_sigma)
    M = torch.zeros(S, device="cuda")
    V = torch.zeros(S, device="cuda")
    wq = torch.zeros(lay.n_pad, dtype=torch.int8, device="cuda")
    wsc = torch.zeros(lay.n_pad // B, device="cuda")
    rng = np.random.default_rng(66)
    blocks = np.unique(np.concatenate([[0, nb - 1], rng.integers(0, nb, size=200)]))
    pos = (blocks[:, None] * B + np.arange(B)[None, :]).reshape(-1)
    flat = rank * S + pos
    w = synth.gather_host(F32, wl.seed, tag(BUF_MASTER, wl.cid), flat, wl.master_sigma)
    m, v = np.zeros(pos.size, np.float32), np.zeros(pos.size, np.float32)
    o_wq = np.zeros(pos.size, np.int8)
    o_ws = np.zeros(blocks.size, np.float32)
    for t in (1, 2):
        for k in range(n_dp):
            synth.fill_device(tmp, F32, wl.seed, tag(BUF_GRAD, wl.cid, t, 0, k), rank * S,
                              d.eff_sigma, d.thr, d.outlier_mul)
            zs.zero_q8_quantize(tmp, rows_q[k], rows_s[k])
        zs.zero_shard_step_q8(rows_q, rows_s, S, nb, S, W, M, V, wq, wsc, lay, rank,
                              zs.AdamWHParams(step=t, grad_scale=1.0 / n_dp, **wl.hp))
        qs, ss = [], []
        for k in range(n_dp):
            x = synth.gather_host(F32, wl.seed, tag(BUF_GRAD, wl.cid, t, 0, k), flat, d.eff_sigma,
                                  d.thr, d.outlier_mul)
            q, s = oracle.q8_quantize(x, oracle.FP32)  # whole blocks: the same blocks as the device
            qs.append(q)
            ss.append(s)
        gq, gs = np.stack(qs), np.stack(ss)
        torch.cuda.synchronize()
        dpos = torch.from_numpy(pos).cuda()
        dblk = torch.from_numpy(blocks).cuda()
        for k in range(n_dp):  # the device quantizer on the sampled blocks
            assert np.array_equal(rows_q[k][dpos].cpu().numpy(), gq[k])
            assert _same_f32(rows_s[k][dblk].cpu().numpy(), gs[k])
        oracle.step_q8(gq.reshape(-1), gs.reshape(-1), n_dp, pos.size, blocks.size, pos.size, w, m,
                       v, o_wq, o_ws, t, grad_scale=1.0 / n_dp, **wl.hp)
    assert _same_f32(W[dpos].cpu().numpy(), w) and _same_f32(M[dpos].cpu().numpy(), m)
    assert _same_f32(V[dpos].cpu().numpy(), v)
    assert np.array_equal(wq[dpos + rank * S].cpu().numpy(), o_wq)
    assert _same_f32(wsc[dblk + rank * nb].cpu().numpy(), o_ws)


def test_quantizer_cases_that_tell_the_readings_apart():
    """Blocks in which rint(x * r) and rint(x / s) differ (found by search,
    as in the oracle's pin): the device quantizer gives the oracle's codes,
    those of the division, on every one, for fp32 and bf16 inputs."""
    rng = np.random.default_rng(11)
    blocks = []
    for _ in range(400):
        amax = np.float32(rng.uniform(0.5, 2.0))
        s = amax / np.float32(127.0)
        k = rng.integers(-126, 127, size=4096).astype(np.float32)
        x = ((k + np.float32(0.5)) * s).astype(np.float32)
        x = x + rng.integers(-2, 3, size=x.size).astype(np.float32) * np.spacing(x)
        x = np.clip(x, -amax, amax).astype(np.float32)
        hit = np.nonzero(np.rint(x * (np.float32(127.0) / amax)) != np.rint(x / s))[0]
        if hit.size:
            blk = np.zeros(B, np.float32)
            blk[0] = amax
            blk[1:1 + min(hit.size, B - 1)] = x[hit[:B - 1]]
            blocks.append(blk)
        if len(blocks) >= 64:
            break
    assert len(blocks) >= 16
    xs = np.concatenate(blocks)
    for kind, arr in ((F32, xs), (BF16, oracle.f32_to_bf16(xs))):
        d = _dev(arr, kind)
        q = torch.empty(xs.size, dtype=torch.int8, device="cuda")
        sc = torch.empty(zs.q8_blocks(xs.size), device="cuda")
        zs.zero_q8_quantize(d, q, sc)
        oq, os_ = oracle.q8_quantize(arr, ODT[kind])
        assert np.array_equal(q.cpu().numpy(), oq)
        assert _same_f32(sc.cpu().numpy(), os_)


def _boundary_blocks():
    """Blocks crowded at the code boundaries: for many block scales (random,
    exact powers of two, subnormal), every half-integer boundary's
    neighbourhood in ulps, each block opening with its absmax."""
    from tests.test_q8_code_rule import _scales, neighbourhoods
    tiny = np.float32(2.0 ** -149)
    scales = list(_scales(5, 24)) + [np.float32(127.0), np.float32(1.0),
                                      np.float32(1e-38), np.float32(64) * tiny,
                                      np.float32(63) * tiny, np.float32(2.0 ** -126)]
    out = []
    for amax in scales:
        x = neighbourhoods(amax, 24)
        n = -(-x.size // (B - 1))
        blk = np.full((n, B), amax, np.float32)
        flat = np.full(n * (B - 1), amax, np.float32)
        flat[:x.size] = x
        blk[:, 1:] = flat.reshape(n, B - 1)
        out.append(blk.reshape(-1))
    return np.concatenate(out)


def test_codes_at_every_boundary_through_the_quantizer_and_the_step():
    """The device's codes equal rint(fl(x / s)) at every code boundary of 30
    block scales, dense in ulps (the same neighbourhoods as the CPU check of
    the shortcut rule): through zero_q8_quantize, and through the fused
    8-bit step's quantization of the new master (lr = 0 and no decay leave
    the master as it was, so the step quantizes exactly these values)."""
    xs = _boundary_blocks()
    n = xs.size
    print(f"\n[q8 boundaries] {n} elements", flush=True)
    oq, os_ = oracle.q8_quantize(xs, oracle.FP32)
    d = _dev(xs, F32)
    q = torch.empty(n, dtype=torch.int8, device="cuda")
    sc = torch.empty(zs.q8_blocks(n), device="cuda")
    zs.zero_q8_quantize(d, q, sc)
    got = q.cpu().numpy()
    assert np.array_equal(got, oq), np.nonzero(got != oq)[0][:8]
    assert _same_f32(sc.cpu().numpy(), os_)
    # the step: one row of zero codes, the master the boundary blocks
    lay, _ = zs.zero_flatten_layout([n], 1, B)
    gq = torch.zeros(n, dtype=torch.int8, device="cuda")
    gs = torch.ones(zs.q8_blocks(n), device="cuda")
    W = d.clone()
    M = torch.zeros(n, device="cuda")
    V = torch.zeros(n, device="cuda")
    wq = torch.zeros(lay.n_pad, dtype=torch.int8, device="cuda")
    wsc = torch.zeros(lay.n_pad // B, device="cuda")
    hp = dict(HP, lr=0.0, weight_decay=0.0)
    zs.zero_shard_step_q8(gq, gs, n, zs.q8_blocks(n), n, W, M, V, wq, wsc, lay, 0,
                          zs.AdamWHParams(step=1, grad_scale=1.0, **hp))
    w, m, v = xs.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    o_wq = np.zeros(n, np.int8)
    o_ws = np.zeros(zs.q8_blocks(n), np.float32)
    oracle.step_q8(np.zeros(n, np.int8), np.ones(zs.q8_blocks(n), np.float32), 1, n,
                   zs.q8_blocks(n), n, w, m, v, o_wq, o_ws, 1, grad_scale=1.0, **hp)
    assert np.array_equal(w.view(np.uint32), xs.view(np.uint32))   # the master kept
    assert np.array_equal(o_wq, oq)
    got = wq.cpu().numpy()[:n]
    assert np.array_equal(got, o_wq), np.nonzero(got != o_wq)[0][:8]
    assert _same_f32(wsc.cpu().numpy()[:zs.q8_blocks(n)], o_ws)
    assert _same_f32(W.cpu().numpy(), w)
