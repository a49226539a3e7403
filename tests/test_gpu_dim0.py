"""GPU parity (through the C ABI) of per-parameter dim-0 sharding and fp32
gradient rows ("ZeRO and FSDP", FSDP section: FSDP2 shards every parameter
along its first dimension, packs a unit's shards into one buffer per
collective, and with its mixed-precision policy reduce-scatters gradients
in float32; the fp32 shard is the master).

  - fp32 rows through the reduce (accumulation, flags, sum of squares) and
    the fused step, bit-exact against the oracle at sizes spanning many
    tiles with ragged tails, aligned and unaligned, n_dp in {1, 3, 8, 64};
  - packing per-parameter tensors into each rank's buffer with the dim-0
    segment map (zero_flat_gather) and unpacking it (zero_flat_scatter);
  - an FSDP2-style step of a small model on every rank, equal to the
    oracle's unsharded step bit for bit;
  - the 7B workload at full size (dim-0 layout, 8 ranks, fp32 rows), on
    sampled elements."""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_flatten_amd as zs
from synth import F32, tag
from synth.synth_const import BUF_GRAD, BUF_MASTER
from synth.workloads import gpt2xl_shapes, workload
from tests.gpu_util import check_16, check_f32, host16, hostf

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


def _rows32(n, length, cfg, t=1, sigma=1e-3, thr=0, mul=1.0):
    return np.stack([synth.fill_host(F32, 0, tag(BUF_GRAD, cfg, t, 0, k), 0, length, sigma,
                                     thr, mul) for k in range(n)])


@pytest.mark.parametrize("n_dp", [1, 3, 8, 64])
@pytest.mark.parametrize("lead", [0, 1])  # 1: rows and state off 16-byte alignment
def test_fp32_rows_reduce_bitwise(n_dp, lead):
    length = 1_048_589 if n_dp <= 8 else 131_101
    ld = length + 3
    rows = _rows32(n_dp, ld, 130 + n_dp, sigma=1.0, thr=synth.synth_const.outlier_threshold(0.01),
                   mul=100.0)
    rows[n_dp - 1, length // 2] = np.inf
    flat = np.concatenate([np.zeros(lead, np.float32), rows.reshape(-1)])
    d_rows = torch.from_numpy(flat).cuda()[lead:]
    acc0 = np.zeros(length + lead, np.float32)
    d_acc = torch.from_numpy(acc0).cuda()[lead:]
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ss = torch.zeros(1, dtype=torch.float64, device="cuda")
    o_acc = np.zeros(length, np.float32)
    o_flag = np.zeros(1, np.uint32)
    o_ss = np.zeros(1, np.float64)
    for mb in range(2):
        zs.zero_shard_reduce(d_rows, n_dp, ld, length, d_acc, accumulate=mb > 0, overflow=flag,
                             sumsq=ss if mb == 1 else None)
        oracle.reduce(rows.reshape(-1), oracle.FP32, n_dp, ld, length, o_acc, mb > 0,
                      overflow=o_flag, sumsq=o_ss if mb == 1 else None)
    torch.cuda.synchronize()
    assert check_f32(hostf(d_acc), o_acc, "acc") == 0
    assert int(flag.item()) == int(o_flag[0]) == 1
    # with an infinity in the data both sums are +inf
    assert np.isinf(ss.item()) and np.isinf(o_ss[0])


@pytest.mark.parametrize("n_dp", [1, 3, 8, 64])
@pytest.mark.parametrize("lead", [0, 1])
def test_fp32_rows_fused_step_bitwise(n_dp, lead):
    length = 1_048_589 if n_dp <= 8 else 131_101
    # aligned case: shard a multiple of 4 (vector path); the last step runs
    # as two calls split at S - 5, so both calls end in element-wise tails
    lay, _ = zs.zero_flatten_layout([length * n_dp], n_dp, 4 if lead == 0 else 1)
    S = lay.shard
    rank = n_dp - 1
    ld = S + 4 if lead == 0 else S + 3
    w = synth.fill_host(F32, 0, tag(BUF_MASTER, 131), 0, S, 0.02)
    m, v = np.zeros(S, np.float32), np.zeros(S, np.float32)
    out = np.zeros(S, np.uint16)
    pad = lambda a: np.concatenate([np.zeros(lead, np.float32), a])
    dw, dm, dv = [torch.from_numpy(pad(a)).cuda()[lead:] for a in (w, m, v)]
    wf = torch.zeros(lay.n_pad + lead, dtype=torch.bfloat16, device="cuda")[lead:]
    for t in (1, 2, 3):
        rows = _rows32(n_dp, ld, 132 + n_dp, t=t)
        d_rows = torch.from_numpy(pad(rows.reshape(-1))).cuda()[lead:]
        ss = torch.zeros(1, dtype=torch.float64, device="cuda")
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        hp = zs.AdamWHParams(step=t, grad_scale=1.0 / n_dp, **HP)
        if t < 3:
            zs.zero_shard_step(d_rows, ld, S, dw, dm, dv, wf, lay, rank, hp, overflow=flag,
                               sumsq=ss)
        else:
            cut = S - 5
            zs.zero_shard_step(d_rows, ld, cut, dw, dm, dv, wf, lay, rank, hp, overflow=flag,
                               sumsq=ss)
            zs.zero_shard_step(d_rows[cut:], ld, S - cut, dw[cut:], dm[cut:], dv[cut:], wf, lay,
                               rank, hp, shard_off=cut, overflow=flag, sumsq=ss)
        o_ss = np.zeros(1, np.float64)
        oracle.step(rows.reshape(-1), oracle.FP32, n_dp, ld, S, w, m, v, out, oracle.BF16, t,
                    grad_scale=1.0 / n_dp, sumsq=o_ss, **HP)
        torch.cuda.synchronize()
        assert int(flag.item()) == 0
        assert abs(ss.item() - o_ss[0]) <= 1e-9 * o_ss[0]
    diff = check_f32(hostf(dw), w, "master") + check_f32(hostf(dm), m, "m")
    diff += check_f32(hostf(dv), v, "v")
    diff += check_16(host16(wf)[rank * S:(rank + 1) * S], out, 0, "weights")
    assert diff == 0


def _pieces_for(tensors, segs):
    return [(tensors[t][toff:toff + ln], soff) for t, toff, soff, ln in segs if t >= 0]


def test_pack_and_unpack_with_the_dim0_segments():
    """GPT-2-XL's parameter shapes scaled down 16x on dim 1 (so that 50257
    and 6400 rows leave padding at 8 ranks): every rank's packed buffer from
    the per-parameter tensors, then unpacked back."""
    shapes = [(r, max(1, c // 16)) for r, c in gpt2xl_shapes()]
    n_dp = 8
    lay, offs, chunk = zs.zero_dim0_layout(shapes, n_dp, 8)
    tensors_h = [synth.fill_host(F32, 1, tag(BUF_MASTER, 133, i), 0, r * c, 0.02)
                 for i, (r, c) in enumerate(shapes)]
    tensors = [torch.from_numpy(t).cuda() for t in tensors_h]
    packed = []
    for rank in range(n_dp):
        segs = zs.zero_dim0_segments(lay, shapes, rank)
        buf = torch.full((lay.shard,), float("nan"), device="cuda")
        zs.zero_flat_gather(_pieces_for(tensors, segs), lay.shard, 0, buf)
        want = np.full(lay.shard, np.nan, np.float32)
        for t, toff, soff, ln in oracle.dim0_segments(shapes, n_dp, rank, 8):
            want[soff:soff + ln] = 0.0 if t < 0 else tensors_h[t][toff:toff + ln]
        got = buf.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"rank {rank}"
        packed.append(buf)
    back = [torch.full((r * c,), float("nan"), device="cuda") for r, c in shapes]
    for rank in range(n_dp):
        segs = zs.zero_dim0_segments(lay, shapes, rank)
        zs.zero_flat_scatter(packed[rank], 0, _pieces_for(back, segs))
    for b, t in zip(back, tensors_h):
        assert np.array_equal(b.cpu().numpy().view(np.uint32), t.view(np.uint32))


def test_fsdp2_style_step_equals_the_unsharded_step():
    """A small model (GPT-2-like shapes with ragged first dimensions) on 4
    ranks: each rank packs the 4 contributors' fp32 gradients for its
    parameters' rows (the reduce-scatter's inputs), steps its fp32 master
    shard and casts into its slot of the bf16 all-gather buffer.  Unpacked,
    every rank's master, m, v and the gathered weights equal the oracle's
    step on the whole (unsharded) parameter vector, bit for bit."""
    shapes = [(1003, 64), (64, 1), (64, 192), (192, 1), (257, 64), (64, 1), (7, 3)]
    n_dp, cfg = 4, 134
    lay, offs, _ = zs.zero_dim0_layout(shapes, n_dp, 4)
    numel = [r * c for r, c in shapes]
    n = sum(numel)
    flat_off = np.concatenate([[0], np.cumsum(numel)[:-1]])
    w_full = synth.fill_host(F32, 0, tag(BUF_MASTER, cfg), 0, n, 0.02)
    m_full, v_full = np.zeros(n, np.float32), np.zeros(n, np.float32)
    wout_full = np.zeros(n, np.uint16)
    as_tensors = lambda flat: [torch.from_numpy(flat[o:o + k].copy()).cuda()
                               for o, k in zip(flat_off, numel)]
    segs = [zs.zero_dim0_segments(lay, shapes, r) for r in range(n_dp)]
    masters = []
    for r in range(n_dp):
        buf = torch.empty(lay.shard, device="cuda")
        zs.zero_flat_gather(_pieces_for(as_tensors(w_full), segs[r]), lay.shard, 0, buf)
        masters.append(buf)
    ms = [torch.zeros(lay.shard, device="cuda") for _ in range(n_dp)]
    vs = [torch.zeros(lay.shard, device="cuda") for _ in range(n_dp)]
    ag = torch.zeros(lay.n_pad, dtype=torch.bfloat16, device="cuda")  # all-gather buffer
    for t in (1, 2):
        grads = _rows32(n_dp, n, cfg, t=t)  # contributor k's full fp32 gradient
        g_tensors = [as_tensors(grads[k]) for k in range(n_dp)]
        for r in range(n_dp):
            rows = torch.empty((n_dp, lay.shard), device="cuda")
            for k in range(n_dp):
                zs.zero_flat_gather(_pieces_for(g_tensors[k], segs[r]), lay.shard, 0, rows[k])
            zs.zero_shard_step(rows, lay.shard, lay.shard, masters[r], ms[r], vs[r], ag, lay, r,
                               zs.AdamWHParams(step=t, grad_scale=1.0 / n_dp, **HP))
        oracle.step(grads.reshape(-1), oracle.FP32, n_dp, n, n, w_full, m_full, v_full,
                    wout_full, oracle.BF16, t, grad_scale=1.0 / n_dp, **HP)
    torch.cuda.synchronize()
    for arr, ref in ((masters, w_full), (ms, m_full), (vs, v_full)):
        back = [torch.full((k,), float("nan"), device="cuda") for k in numel]
        for r in range(n_dp):
            zs.zero_flat_scatter(arr[r], 0, _pieces_for(back, segs[r]))
        got = torch.cat(back).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # the all-gather buffer, unpacked per rank, is the cast of the new master
    ag16 = ag.view(torch.int16)
    back = [torch.zeros(k, dtype=torch.int16, device="cuda") for k in numel]
    for r in range(n_dp):
        zs.zero_flat_scatter(ag16[r * lay.shard:(r + 1) * lay.shard], 0, _pieces_for(back, segs[r]))
    got = torch.cat(back).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, wout_full)


def test_dim0_fp32_workload_full_size():
    """The 7B list in the dim-0 layout over 8 ranks (842,301,952 packed
    elements per rank), rank 1, fp32 gradient rows with 1 % outliers x100,
    t = 1..3, against the oracle on sampled elements."""
    wl = workload(5)
    lay, _, _ = zs.zero_dim0_layout(wl.shapes, wl.n_dp)
    S, n_dp, rank = lay.shard, wl.n_dp, wl.rank
    print(f"\n[full] dim-0 fp32 rows S={S} n_dp={n_dp} rank={rank}", flush=True)
    d = wl.grad
    slab = torch.empty((n_dp, S), dtype=torch.float32, device="cuda")
    W = torch.empty(S, device="cuda")
    synth.fill_device(W, F32, wl.seed, tag(BUF_MASTER, wl.cid), rank * S, wl.master_sigma)
    M = torch.zeros(S, device="cuda")
    V = torch.zeros(S, device="cuda")
    wf = torch.zeros(lay.n_pad, dtype=torch.bfloat16, device="cuda")
    for t in wl.steps:
        for k in range(n_dp):
            synth.fill_device(slab[k], F32, wl.seed, tag(BUF_GRAD, wl.cid, t, 0, k), rank * S,
                              d.eff_sigma, d.thr, d.outlier_mul)
        zs.zero_shard_step(slab, S, S, W, M, V, wf, lay, rank,
                           zs.AdamWHParams(step=t, grad_scale=1.0 / n_dp, **wl.hp))
    torch.cuda.synchronize()
    rng = np.random.default_rng(55)
    idx = np.unique(np.concatenate([np.arange(1024), S - 1024 + np.arange(1024),
                                    rng.integers(0, S, size=20000)])).astype(np.int64)
    pos = rank * S + idx
    w = synth.gather_host(F32, wl.seed, tag(BUF_MASTER, wl.cid), pos, wl.master_sigma)
    m, v = np.zeros(idx.size, np.float32), np.zeros(idx.size, np.float32)
    out = np.zeros(idx.size, np.uint16)
    for t in wl.steps:
        rows = np.stack([synth.gather_host(F32, wl.seed, tag(BUF_GRAD, wl.cid, t, 0, k), pos,
                                           d.eff_sigma, d.thr, d.outlier_mul)
                         for k in range(n_dp)])
        oracle.step(rows.reshape(-1), oracle.FP32, n_dp, idx.size, idx.size, w, m, v, out,
                    oracle.BF16, t, grad_scale=1.0 / n_dp, **wl.hp)
    di = torch.from_numpy(idx).cuda()
    diff = check_f32(W[di].cpu().numpy(), w, "master") + check_f32(M[di].cpu().numpy(), m, "m")
    diff += check_f32(V[di].cpu().numpy(), v, "v")
    got = wf.view(torch.int16)[di + rank * S].cpu().numpy().view(np.uint16)
    diff += check_16(got, out, 0, "weights")
    assert diff == 0
