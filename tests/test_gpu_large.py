"""Ranges longer than one launch: a dispatch counts its grid in work-items in
32 bits, so the one-shot kernels cover at most 2^31 elements per launch and
the entry points issue consecutive launches; the grid-stride kernels cap
their grid and loop; the copy kernel splits copies of more than 2^32 bytes.
Each test runs one entry point over a range just past such a boundary and
checks, against the oracle, sampled elements on both sides of every boundary,
the ragged tail and random positions (whole blocks for the 8-bit path).

The arithmetic is the sharded step of "ZeRO and FSDP" (A sharded Adam step)
and its 8-bit reading (FSDP section, ZeRO++); the copies are the flat
gathers of checkpoint conversion.  Sizes need a few tens of GB of HBM."""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_flatten_amd as zs
from synth import BF16, F32, tag
from synth.synth_const import BUF_GRAD, BUF_MASTER
from tests.gpu_util import check_16, check_f32

pytestmark = pytest.mark.gpu

L = 1 << 31                      # elements per launch of a one-shot kernel
B = zs.ZERO_Q8_BLOCK
HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
CID = 170                        # stream tags of this file


def _points(n, marks, seed, k=4000):
    rng = np.random.default_rng(seed)
    pts = [np.arange(0, 64), np.arange(n - 64, n), rng.integers(0, n, size=k)]
    for p in marks:
        pts.append(np.arange(max(0, p - 40), min(n, p + 40)))
    return np.unique(np.concatenate(pts)).astype(np.int64)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _same_f32(a, b):
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32))


def test_step_across_launches():
    """The fused step (n_dp = 1, bf16 row) over 2^31 + 4099 elements: the
    quad kernel in two launches, then a 3-element tail; step 1 plain, step 2
    with the overflow flag and the sum of squares (partials from both
    launches and the tail, then the fixed-order finish)."""
    n = L + 4099
    print(f"\n[large] step n={n}", flush=True)
    lay, _ = zs.zero_flatten_layout([n], 1)
    g = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    W = torch.empty(n, device="cuda")
    synth.fill_device(W, F32, 1, tag(BUF_MASTER, CID), 0, 0.02)
    M = torch.zeros(n, device="cuda")
    V = torch.zeros(n, device="cuda")
    wf = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    idx = _points(n, [L, n - 3], 1)
    w = synth.gather_host(F32, 1, tag(BUF_MASTER, CID), idx, 0.02)
    m, v = np.zeros(idx.size, np.float32), np.zeros(idx.size, np.float32)
    out = np.zeros(idx.size, np.uint16)
    for t in (1, 2):
        synth.fill_device(g, BF16, 1, tag(BUF_GRAD, CID, t), 0, 1e-3)
        hp = zs.AdamWHParams(step=t, grad_scale=1.0, **HP)
        if t == 1:
            zs.zero_shard_step(g, n, n, W, M, V, wf, lay, 0, hp)
        else:
            flag = torch.zeros(1, dtype=torch.int32, device="cuda")
            ss = torch.zeros(1, dtype=torch.float64, device="cuda")
            zs.zero_shard_step(g, n, n, W, M, V, wf, lay, 0, hp, overflow=flag, sumsq=ss)
            # the sum of squares by its definition, in fp64 over pieces
            ref = sum(float((g[o:o + (1 << 28)].float().double() ** 2).sum())
                      for o in range(0, n, 1 << 28))
            assert int(flag.item()) == 0
            assert abs(ss.item() - ref) <= 1e-9 * ref
        rows = synth.gather_host(BF16, 1, tag(BUF_GRAD, CID, t), idx, 1e-3)
        oracle.step(rows, oracle.BF16, 1, idx.size, idx.size, w, m, v, out, oracle.BF16, t,
                    grad_scale=1.0, **HP)
    di = torch.from_numpy(idx).cuda()
    diff = check_f32(W[di].cpu().numpy(), w, "master") + check_f32(M[di].cpu().numpy(), m, "m")
    diff += check_f32(V[di].cpu().numpy(), v, "v")
    diff += check_16(wf.view(torch.int16)[di].cpu().numpy().view(np.uint16), out, 0, "weights")
    assert diff == 0
    del g, W, M, V, wf
    _free()


def test_grid_stride_kernels_loop():
    """Unaligned buffers take the element-per-thread kernels, whose grid is
    capped at 2^20 workgroups of 256 (2^28 threads): over 2^28 + 777
    elements every thread past the cap's reach loops once.  The reduce, the
    AdamW and the fused step, each against the oracle."""
    n = (1 << 28) + 777
    print(f"\n[large] grid-stride n={n}", flush=True)
    lay, _ = zs.zero_flatten_layout([n], 1)
    gb = torch.empty(n + 1, dtype=torch.bfloat16, device="cuda")
    g = gb[1:]                   # 2-byte aligned: the element path
    synth.fill_device(g, BF16, 2, tag(BUF_GRAD, CID, 9), 0, 1e-3)
    ab = torch.zeros(n + 1, device="cuda")
    acc = ab[1:]
    zs.zero_shard_reduce(g, 1, n, n, acc)
    W = torch.empty(n + 1, device="cuda")[1:]
    synth.fill_device(W, F32, 2, tag(BUF_MASTER, CID), 0, 0.02)
    M = torch.zeros(n + 1, device="cuda")[1:]
    V = torch.zeros(n + 1, device="cuda")[1:]
    wf = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    hp = zs.AdamWHParams(step=1, grad_scale=1.0, **HP)
    zs.zero_shard_adamw(acc, W, M, V, wf, lay, 0, hp)
    W2 = torch.empty(n + 1, device="cuda")[1:]
    synth.fill_device(W2, F32, 2, tag(BUF_MASTER, CID), 0, 0.02)
    M2 = torch.zeros(n + 1, device="cuda")[1:]
    V2 = torch.zeros(n + 1, device="cuda")[1:]
    wf2 = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    zs.zero_shard_step(g, n, n, W2, M2, V2, wf2, lay, 0, hp)
    idx = _points(n, [1 << 28], 2)
    rows = synth.gather_host(BF16, 2, tag(BUF_GRAD, CID, 9), idx, 1e-3)
    a = np.zeros(idx.size, np.float32)
    oracle.reduce(rows, oracle.BF16, 1, idx.size, idx.size, a, False)
    w0 = synth.gather_host(F32, 2, tag(BUF_MASTER, CID), idx, 0.02)
    w, m, v = w0.copy(), np.zeros(idx.size, np.float32), np.zeros(idx.size, np.float32)
    out = np.zeros(idx.size, np.uint16)
    oracle.adamw(a, w, m, v, out, oracle.BF16, idx.size, 1, grad_scale=1.0, **HP)
    w2, m2, v2 = w0.copy(), np.zeros(idx.size, np.float32), np.zeros(idx.size, np.float32)
    out2 = np.zeros(idx.size, np.uint16)
    oracle.step(rows, oracle.BF16, 1, idx.size, idx.size, w2, m2, v2, out2, oracle.BF16, 1,
                grad_scale=1.0, **HP)
    di = torch.from_numpy(idx).cuda()
    diff = check_f32(acc[di].cpu().numpy(), a, "acc")
    for (dW, dM, dV, dwf), (ow, om, ov, oo) in (((W, M, V, wf), (w, m, v, out)),
                                                ((W2, M2, V2, wf2), (w2, m2, v2, out2))):
        diff += check_f32(dW[di].cpu().numpy(), ow, "master")
        diff += check_f32(dM[di].cpu().numpy(), om, "m") + check_f32(dV[di].cpu().numpy(), ov, "v")
        diff += check_16(dwf.view(torch.int16)[di].cpu().numpy().view(np.uint16), oo, 0, "weights")
    assert diff == 0
    del gb, g, ab, acc, W, M, V, wf, W2, M2, V2, wf2
    _free()


def _blocks(nb, marks, seed, k=300):
    rng = np.random.default_rng(seed)
    b = [np.arange(0, 2), np.arange(nb - 2, nb), rng.integers(0, nb, size=k)]
    for p in marks:
        b.append(np.arange(max(0, p - 2), min(nb, p + 2)))
    return np.unique(np.concatenate(b)).astype(np.int64)


def _block_positions(blocks, n):
    pos = (blocks[:, None] * B + np.arange(B)[None, :]).reshape(-1)
    return pos[pos < n]


def test_codec_across_launches():
    """Quantize (fp32 in) and dequantize (to bf16: the paired-block kernel;
    to fp32: the quad kernel) over 2^31 + 300 elements: two launches each,
    the last block 44 elements long."""
    n = L + 300
    print(f"\n[large] codec n={n}", flush=True)
    nb = zs.q8_blocks(n)
    x = torch.empty(n, device="cuda")
    synth.fill_device(x, F32, 3, tag(BUF_GRAD, CID, 3), 0, 1e-3)
    q = torch.empty(n, dtype=torch.int8, device="cuda")
    s = torch.empty(nb, device="cuda")
    zs.zero_q8_quantize(x, q, s)
    del x
    _free()
    yb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    zs.zero_q8_dequantize(q, s, yb)
    blocks = _blocks(nb, [L // B], 3)
    pos = _block_positions(blocks, n)
    xs = synth.gather_host(F32, 3, tag(BUF_GRAD, CID, 3), pos, 1e-3)
    # the sampled blocks one after another, the short last block at the end:
    # the oracle's blocks of the concatenation are the device's blocks
    oq, os_ = oracle.q8_quantize(xs, oracle.FP32)
    dp = torch.from_numpy(pos).cuda()
    assert np.array_equal(q[dp].cpu().numpy(), oq)
    assert _same_f32(s[torch.from_numpy(blocks).cuda()].cpu().numpy(), os_)
    ob = oracle.q8_dequantize(oq, os_, oracle.BF16)
    assert check_16(yb.view(torch.int16)[dp].cpu().numpy().view(np.uint16), ob, oracle.BF16,
                    "bf16") == 0
    del yb
    _free()
    yf = torch.empty(n, device="cuda")
    zs.zero_q8_dequantize(q, s, yf)
    of = oracle.q8_dequantize(oq, os_, oracle.FP32)
    assert _same_f32(yf[dp].cpu().numpy(), of)
    del q, s, yf
    _free()


def test_q8_step_across_launches():
    """The fused 8-bit step (n_dp = 1) over a 2^31 + 512-element shard: two
    launches, the second of two blocks; codes quantized on the device from
    fp32 draws, checked on whole sampled blocks."""
    n = L + 2 * B
    print(f"\n[large] q8 step n={n}", flush=True)
    lay, _ = zs.zero_flatten_layout([n], 1, B)
    assert lay.shard == n
    nb = n // B
    x = torch.empty(n, device="cuda")
    synth.fill_device(x, F32, 4, tag(BUF_GRAD, CID, 4), 0, 1e-3)
    gq = torch.empty(n, dtype=torch.int8, device="cuda")
    gs = torch.empty(nb, device="cuda")
    zs.zero_q8_quantize(x, gq, gs)
    W = x                        # reuse the draw buffer for the master
    synth.fill_device(W, F32, 4, tag(BUF_MASTER, CID), 0, 0.02)
    M = torch.zeros(n, device="cuda")
    V = torch.zeros(n, device="cuda")
    wq = torch.zeros(n, dtype=torch.int8, device="cuda")
    wsc = torch.zeros(nb, device="cuda")
    zs.zero_shard_step_q8(gq, gs, n, nb, n, W, M, V, wq, wsc, lay, 0,
                          zs.AdamWHParams(step=1, grad_scale=1.0, **HP))
    blocks = _blocks(nb, [L // B], 4)
    pos = _block_positions(blocks, n)
    xs = synth.gather_host(F32, 4, tag(BUF_GRAD, CID, 4), pos, 1e-3)
    q, sc = oracle.q8_quantize(xs, oracle.FP32)      # whole blocks: the device's blocks
    w = synth.gather_host(F32, 4, tag(BUF_MASTER, CID), pos, 0.02)
    m, v = np.zeros(pos.size, np.float32), np.zeros(pos.size, np.float32)
    o_wq, o_ws = np.zeros(pos.size, np.int8), np.zeros(blocks.size, np.float32)
    oracle.step_q8(q, sc, 1, pos.size, blocks.size, pos.size, w, m, v, o_wq, o_ws, 1,
                   grad_scale=1.0, **HP)
    dp, db = torch.from_numpy(pos).cuda(), torch.from_numpy(blocks).cuda()
    assert np.array_equal(gq[dp].cpu().numpy(), q) and _same_f32(gs[db].cpu().numpy(), sc)
    assert _same_f32(W[dp].cpu().numpy(), w) and _same_f32(M[dp].cpu().numpy(), m)
    assert _same_f32(V[dp].cpu().numpy(), v)
    assert np.array_equal(wq[dp].cpu().numpy(), o_wq) and _same_f32(wsc[db].cpu().numpy(), o_ws)
    del x, W, gq, gs, M, V, wq, wsc
    _free()


@pytest.mark.parametrize("phase", [0, 1])
def test_copy_longer_than_a_segment(phase):
    """A flat gather of one fp32 piece of 2^30 + 1001 elements (just over
    2^32 bytes: two segments), with the destination at the source's
    alignment phase or 4 bytes off it; bitwise on the device, the zero-filled
    indices past the piece included."""
    n = (1 << 30) + 1001
    print(f"\n[large] copy n={n} phase={phase}", flush=True)
    src = torch.empty(n, device="cuda")
    synth.fill_device(src, F32, 5, tag(BUF_MASTER, CID, 5), 0, 1.0)
    buf = torch.full((n + 17 + phase,), 7.0, device="cuda")
    dst = buf[phase:phase + n + 16]
    zs.zero_flat_gather([(src, 0)], n + 16, 0, dst)
    assert torch.equal(dst[:n].view(torch.int32), src.view(torch.int32))
    assert bool((dst[n:] == 0).all())
    if phase:
        assert float(buf[0].item()) == 7.0
    assert float(buf[-1].item()) == 7.0
    del src, buf, dst
    _free()
