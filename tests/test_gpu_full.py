"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times: every step of each workload runs on the GPU over the whole
shard; the oracle recomputes sampled elements one by one (their inputs are
regenerated on the host from the same counter-based streams) through the
same sequence of steps.  Bytes outside the rank's slot of the full weight
buffer are checked on the device to keep their canary value.

Workloads (parameter lists from synth.workloads):
  GPT-2-XL-shaped, n_dp = 1 (1,557,611,200 parameters; 5 warm-up steps, t=6)
  Llama-shaped 7B, n_dp = 8, rank 1 (842,301,952-parameter shard; t = 1..10;
      bf16 gradients with 1% outliers x100), and rank 7 (slot beyond 2^32
      elements of the weight buffer)
  Llama-shaped 7B, n_dp = 64 (105,287,744-parameter shard; 9 warm-up steps, t=10)
  Llama-shaped 7B, n_dp = 8, fp16 gradients x 65536, 4 micro-batches reduced
      into an fp32 accumulator, unscaled, AdamW gated on the overflow flag
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_flatten_amd as zs
from synth import F32, F16
from synth.synth_const import BUF_GRAD, BUF_MASTER
from synth.workloads import workload
from tests.gpu_util import check_16, check_f32

pytestmark = pytest.mark.gpu

CANARY = 0x5A5A


def _sample(S, n=20000, seed=0):
    rng = np.random.default_rng(seed)
    pts = [np.arange(0, min(S, 1024)), np.arange(max(0, S - 1024), S),
           rng.integers(0, S, size=n)]
    for p in (1 << 20, 1 << 24, 1 << 28, 1 << 29, 1 << 30, 1 << 31):
        if p < S:
            pts.append(np.arange(max(0, p - 8), min(S, p + 8)))
    return np.unique(np.concatenate(pts)).astype(np.int64)


def _fill_rows(slab, wl, step, micro, start):
    d = wl.grad
    for k in range(slab.shape[0]):
        synth.fill_device(slab[k], d.kind, wl.seed, synth.tag(BUF_GRAD, wl.cid, step, micro, k),
                          start, d.eff_sigma, d.thr, d.outlier_mul)


def _gather_rows(wl, step, micro, flat_idx):
    d = wl.grad
    return np.stack([synth.gather_host(d.kind, wl.seed, synth.tag(BUF_GRAD, wl.cid, step, micro, k),
                                       flat_idx, d.eff_sigma, d.thr, d.outlier_mul)
                     for k in range(wl.n_dp)])


def _canaries_ok(wf, lo, hi):
    c = torch.tensor(CANARY, dtype=torch.int16, device=wf.device)
    v = wf.view(torch.int16)
    return bool((v[:lo] == c).all()) and bool((v[hi:] == c).all())


@pytest.mark.parametrize("cid,rank,steps", [
    (2, 1, None),            # 7B n_dp=8 rank 1, t = 1..10 (the benchmark's workload)
    (2, 7, (1, 2)),          # last rank: slot above 2^32 elements
    (1, 0, None),            # GPT-2-XL n_dp=1, 5 warm-up steps then t = 6
    (3, 1, None),            # 7B n_dp=64, 9 warm-up steps then t = 10
])
def test_fused_step_full_size(cid, rank, steps):
    wl = workload(cid)
    lay, _ = zs.zero_flatten_layout(wl.numels, wl.n_dp)
    S, n_dp = lay.shard, wl.n_dp
    ts = tuple(range(1, wl.warmup_steps + 1)) + wl.steps if steps is None else steps
    print(f"\n[full] config {cid} rank {rank} S={S} n_dp={n_dp} steps={ts}", flush=True)
    dev = torch.device("cuda")
    tdt = torch.bfloat16 if wl.grad.kind == synth.BF16 else torch.float16
    slab = torch.empty((n_dp, S), dtype=tdt, device=dev)
    W = torch.empty(S, dtype=torch.float32, device=dev)
    synth.fill_device(W, F32, wl.seed, synth.tag(BUF_MASTER, cid), rank * S, wl.master_sigma)
    M = torch.zeros(S, dtype=torch.float32, device=dev)
    V = torch.zeros(S, dtype=torch.float32, device=dev)
    wf = torch.full((lay.n_pad,), CANARY, dtype=torch.int16, device=dev).view(torch.bfloat16)
    for t in ts:
        _fill_rows(slab, wl, t, 0, rank * S)
        hp = zs.AdamWHParams(step=t, grad_scale=1.0 / n_dp, **wl.hp)
        zs.zero_shard_step(slab, S, S, W, M, V, wf, lay, rank, hp)
    torch.cuda.synchronize()
    # oracle on the sampled elements, through the same steps
    idx = _sample(S, seed=cid * 10 + rank)
    flat = rank * S + idx
    w = synth.gather_host(F32, wl.seed, synth.tag(BUF_MASTER, cid), flat, wl.master_sigma)
    m = np.zeros(idx.size, np.float32)
    v = np.zeros(idx.size, np.float32)
    out = np.zeros(idx.size, np.uint16)
    gdt = oracle.BF16 if wl.grad.kind == synth.BF16 else oracle.FP16
    for t in ts:
        rows = _gather_rows(wl, t, 0, flat)
        oracle.step(rows, gdt, n_dp, idx.size, idx.size, w, m, v, out, oracle.BF16, t,
                    grad_scale=1.0 / n_dp, **wl.hp)
    di = torch.from_numpy(idx).to(dev)
    diff = check_f32(W[di].cpu().numpy(), w, "master")
    diff += check_f32(M[di].cpu().numpy(), m, "m")
    diff += check_f32(V[di].cpu().numpy(), v, "v")
    got = wf.view(torch.int16)[di + rank * S].cpu().numpy().view(np.uint16)
    diff += check_16(got, out, 0, "weights")
    assert diff == 0, f"{diff} sampled values differ from the oracle bitwise"
    assert _canaries_ok(wf, rank * S, (rank + 1) * S)


def test_accumulation_full_size():
    """Stage-2 accumulation at full size: 4 micro-batches of 8 fp16 rows
    (loss scale 65536) reduced into an fp32 shard accumulator, AdamW after
    micro-batch 4, gated on the overflow flag (none here)."""
    wl = workload(4)
    lay, _ = zs.zero_flatten_layout(wl.numels, wl.n_dp)
    S, n_dp, rank, micro = lay.shard, wl.n_dp, wl.rank, wl.micro_batches
    print(f"\n[full] config 4 rank {rank} S={S} micro={micro}", flush=True)
    dev = torch.device("cuda")
    slab = torch.empty((n_dp, S), dtype=torch.float16, device=dev)
    acc = torch.empty(S, dtype=torch.float32, device=dev)
    W = torch.empty(S, dtype=torch.float32, device=dev)
    synth.fill_device(W, F32, wl.seed, synth.tag(BUF_MASTER, 4), rank * S, wl.master_sigma)
    M = torch.zeros(S, dtype=torch.float32, device=dev)
    V = torch.zeros(S, dtype=torch.float32, device=dev)
    wf = torch.full((lay.n_pad,), CANARY, dtype=torch.int16, device=dev).view(torch.bfloat16)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    scale = 1.0 / (n_dp * wl.loss_scale * micro)
    for mb in range(micro):
        _fill_rows(slab, wl, 1, mb, rank * S)
        zs.zero_shard_reduce(slab, n_dp, S, S, acc, accumulate=mb > 0, overflow=flag)
    zs.zero_shard_adamw(acc, W, M, V, wf, lay, rank, zs.AdamWHParams(step=1, grad_scale=scale, **wl.hp),
                        skip=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    idx = _sample(S, seed=44)
    flat = rank * S + idx
    a = np.zeros(idx.size, np.float32)
    o_flag = np.zeros(1, np.uint32)
    for mb in range(micro):
        oracle.reduce(_gather_rows(wl, 1, mb, flat), oracle.FP16, n_dp, idx.size, idx.size, a,
                      mb > 0, overflow=o_flag)
    w = synth.gather_host(F32, wl.seed, synth.tag(BUF_MASTER, 4), flat, wl.master_sigma)
    m = np.zeros(idx.size, np.float32)
    v = np.zeros(idx.size, np.float32)
    out = np.zeros(idx.size, np.uint16)
    oracle.adamw(a, w, m, v, out, oracle.BF16, idx.size, 1, grad_scale=scale, skip=o_flag, **wl.hp)
    di = torch.from_numpy(idx).to(dev)
    diff = check_f32(acc[di].cpu().numpy(), a, "acc")
    diff += check_f32(W[di].cpu().numpy(), w, "master") + check_f32(M[di].cpu().numpy(), m, "m")
    diff += check_f32(V[di].cpu().numpy(), v, "v")
    diff += check_16(wf.view(torch.int16)[di + rank * S].cpu().numpy().view(np.uint16), out, 0, "w")
    assert diff == 0
    assert _canaries_ok(wf, rank * S, (rank + 1) * S)


def test_sum_of_squares_full_size():
    """The optional shard sum of squares at full size, against a float64 sum
    of the oracle's g^2 over a sampled slice and the device-side float64
    sum of the same squares (an order-independent reference)."""
    wl = workload(2)
    lay, _ = zs.zero_flatten_layout(wl.numels, wl.n_dp)
    S, n_dp, rank = lay.shard, wl.n_dp, wl.rank
    dev = torch.device("cuda")
    slab = torch.empty((n_dp, S), dtype=torch.bfloat16, device=dev)
    _fill_rows(slab, wl, 1, 0, rank * S)
    W = torch.zeros(S, dtype=torch.float32, device=dev)
    M = torch.zeros(S, dtype=torch.float32, device=dev)
    V = torch.zeros(S, dtype=torch.float32, device=dev)
    wf = torch.zeros(lay.n_pad, dtype=torch.bfloat16, device=dev)
    ss = torch.zeros(1, dtype=torch.float64, device=dev)
    ovf = torch.zeros(1, dtype=torch.int32, device=dev)
    zs.zero_shard_step(slab, S, S, W, M, V, wf, lay, rank,
                       zs.AdamWHParams(step=1, grad_scale=1.0 / n_dp, **wl.hp), overflow=ovf, sumsq=ss)
    # reference: sum of the reduced gradient's squares, with the reduce done
    # by the oracle's order on the device's rows (fp32 left-to-right sum in
    # torch on the device, then float64 squares)
    a = slab[0].float()
    for k in range(1, n_dp):
        a = a + slab[k].float()
    g = (a * (1.0 / n_dp)).double()
    ref = float((g * g).sum().item())
    torch.cuda.synchronize()
    assert int(ovf.item()) == 0
    assert abs(ss.item() - ref) <= 1e-9 * ref


def test_controlled_fp16_step_full_size():
    """Configuration 7 at full size: 4 micro-batches of 8 fp16 rows reduced
    into the fp32 accumulator, the last reduce also summing squares; AdamW
    with the skip flag, clipping to a norm it must clip to, and the
    device-resident loss scale; then the scale update.  The accumulator and
    the state against the oracle on sampled elements (bit for bit, the
    oracle given the device's sum of squares), the device's sum of squares
    against a float64 sum of the accumulator's squares over the whole shard
    (order-independent reference)."""
    wl = workload(7)
    lay, _ = zs.zero_flatten_layout(wl.numels, wl.n_dp)
    S, n_dp, rank, micro = lay.shard, wl.n_dp, wl.rank, wl.micro_batches
    print(f"\n[full] config 7 rank {rank} S={S} micro={micro}", flush=True)
    dev = torch.device("cuda")
    slab = torch.empty((n_dp, S), dtype=torch.float16, device=dev)
    acc = torch.empty(S, dtype=torch.float32, device=dev)
    W = torch.empty(S, dtype=torch.float32, device=dev)
    synth.fill_device(W, F32, wl.seed, synth.tag(BUF_MASTER, 7), rank * S, wl.master_sigma)
    M = torch.zeros(S, dtype=torch.float32, device=dev)
    V = torch.zeros(S, dtype=torch.float32, device=dev)
    wf = torch.full((lay.n_pad,), CANARY, dtype=torch.int16, device=dev).view(torch.bfloat16)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    ss = torch.zeros(1, dtype=torch.float64, device=dev)
    dls = zs.new_loss_scale(wl.loss_scale)
    for mb in range(micro):
        _fill_rows(slab, wl, 1, mb, rank * S)
        zs.zero_shard_reduce(slab, n_dp, S, S, acc, accumulate=mb > 0, overflow=flag,
                             sumsq=ss if mb == micro - 1 else None)
    torch.cuda.synchronize()
    # the whole shard's sum of squares, float64, in chunks on the device
    ref = 0.0
    for lo in range(0, S, 1 << 27):
        a = acc[lo:lo + (1 << 27)].double()
        ref += float((a * a).sum().item())
    d_ss = float(ss.item())
    assert abs(d_ss - ref) <= 1e-9 * ref
    # the clip must bite: norm = sqrt(ss) * s with s = 1 / (n_dp * micro * scale)
    s = 1.0 / (n_dp * micro) / wl.loss_scale
    max_norm = 0.5 * (d_ss ** 0.5) * s
    hp = zs.AdamWHParams(step=1, grad_scale=1.0 / (n_dp * micro), **wl.hp)
    zs.zero_shard_adamw_ex(acc, W, M, V, wf, lay, rank, hp, skip=flag, sumsq=ss,
                           max_norm=max_norm, loss_scale=dls)
    zs.zero_loss_scale_update(dls, flag, 2.0, 0.5, 2000)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    assert zs.read_loss_scale(dls) == (wl.loss_scale, 1)
    idx = _sample(S, seed=77)
    flat = rank * S + idx
    a = np.zeros(idx.size, np.float32)
    o_flag = np.zeros(1, np.uint32)
    for mb in range(micro):
        oracle.reduce(_gather_rows(wl, 1, mb, flat), oracle.FP16, n_dp, idx.size, idx.size, a,
                      mb > 0, overflow=o_flag)
    assert oracle.clip_coef(d_ss, np.float32(s), max_norm) < 1.0
    w = synth.gather_host(F32, wl.seed, synth.tag(BUF_MASTER, 7), flat, wl.master_sigma)
    m = np.zeros(idx.size, np.float32)
    v = np.zeros(idx.size, np.float32)
    out = np.zeros(idx.size, np.uint16)
    oracle.adamw_ex(a, w, m, v, out, oracle.BF16, idx.size, 1, grad_scale=1.0 / (n_dp * micro),
                    skip=o_flag, sumsq=np.array([d_ss]), max_norm=max_norm,
                    loss_scale=np.array([wl.loss_scale], np.float32), **wl.hp)
    di = torch.from_numpy(idx).to(dev)
    diff = check_f32(acc[di].cpu().numpy(), a, "acc")
    diff += check_f32(W[di].cpu().numpy(), w, "master") + check_f32(M[di].cpu().numpy(), m, "m")
    diff += check_f32(V[di].cpu().numpy(), v, "v")
    diff += check_16(wf.view(torch.int16)[di + rank * S].cpu().numpy().view(np.uint16), out, 0, "w")
    assert diff == 0
    assert _canaries_ok(wf, rank * S, (rank + 1) * S)
