"""Every element of a full-size shard against the oracle ("ZeRO and FSDP",
"A sharded Adam step": rank r's whole shard after the step).

The GPU runs a workload's whole trajectory over the whole shard, in the
launch configuration the benchmark times.  Then the shard is compared chunk
by chunk: for each chunk the oracle replays the same steps on its elements,
on all host cores (the update is element-wise, so each thread takes one
contiguous range of the chunk and the result equals one whole-range call),
and every element of master, m, v and the rank's weight slot must be bit
for bit the oracle's.

Inputs come from the shared seeded generator (synth, which holds none of
the method's arithmetic): the master is drawn on the host; each step's
gradient rows for a chunk are drawn on the device by the generator's device
build, which draws bit-identical values to its host build
(tests/test_gpu_synth.py), and copied to the host for the oracle -- drawing
the 6.7e10 gradient values of a trajectory on the host would take minutes.

Workloads: the Llama-shaped 7B list over n_dp = 8, rank 1 (842,301,952
elements, t = 1..10, the benchmark's workload) and over n_dp = 64, rank 1
(105,287,744 elements, 9 warm-up steps and t = 10); the GPT-2-XL-shaped list
at n_dp = 1 (1,557,611,200 elements, 5 warm-up steps and t = 6); and the 7B
stage-2 accumulation (fp16 rows x 65536, 4 micro-batches reduced into the
fp32 accumulator, AdamW gated on the overflow flag), whose accumulator is
compared too, alone and with global-norm clipping and the device-resident
loss scale; the 7B list in the per-parameter dim-0 layout with fp32
gradient rows (842,301,952 packed elements, t = 1..3); and the 8-bit path
(fp32 draws quantized to int8 blocks on the device, the fused 8-bit step
at t = 1, 2: every code and scale of the last step's rows, of the weight
slot and every element of the state)."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_flatten_amd as zs
from synth import F32
from synth.synth_const import BUF_GRAD, BUF_MASTER
from synth.workloads import workload

pytestmark = pytest.mark.gpu


def _threads():
    return synth.host_threads()


def _oracle_steps(rows_of, ts, w, m, v, out, n_dp, wl):
    """The oracle's steps ts on one chunk (w, m, v, out in place); rows_of(t)
    gives step t's rows as one flat uint16 array of n_dp * chunk elements."""
    n = w.size
    T = _threads()
    cuts = [n * i // T for i in range(T + 1)]
    with ThreadPoolExecutor(max_workers=T) as pool:
        for t in ts:
            flat = rows_of(t)

            def run(i, flat=flat, t=t):
                a, b = cuts[i], cuts[i + 1]
                oracle.step(flat[a:], oracle.BF16, n_dp, n, b - a, w[a:b], m[a:b], v[a:b],
                            out[a:b], oracle.BF16, t, grad_scale=1.0 / n_dp, **wl.hp)
            list(pool.map(run, range(T)))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid,chunk_log2", [(2, 26), (3, 23), (1, 27)])
def test_every_element_of_the_full_shard(cid, chunk_log2):
    wl = workload(cid)
    lay, _ = zs.zero_flatten_layout(wl.numels, wl.n_dp)
    S, n_dp, rank = lay.shard, wl.n_dp, wl.rank
    ts = tuple(range(1, wl.warmup_steps + 1)) + wl.steps
    d = wl.grad
    print(f"\n[full shard] config {cid} rank {rank} S={S} n_dp={n_dp} steps={ts}", flush=True)
    dev = torch.device("cuda")
    slab = torch.empty((n_dp, S), dtype=torch.bfloat16, device=dev)
    W = torch.empty(S, dtype=torch.float32, device=dev)
    synth.fill_device(W, F32, wl.seed, synth.tag(BUF_MASTER, cid), rank * S, wl.master_sigma)
    M = torch.zeros(S, dtype=torch.float32, device=dev)
    V = torch.zeros(S, dtype=torch.float32, device=dev)
    wf = torch.zeros(lay.n_pad, dtype=torch.bfloat16, device=dev)
    for t in ts:
        for k in range(n_dp):
            synth.fill_device(slab[k], d.kind, wl.seed, synth.tag(BUF_GRAD, cid, t, 0, k),
                              rank * S, d.eff_sigma, d.thr, d.outlier_mul)
        zs.zero_shard_step(slab, S, S, W, M, V, wf, lay, rank,
                           zs.AdamWHParams(step=t, grad_scale=1.0 / n_dp, **wl.hp))
    torch.cuda.synchronize()
    del slab
    torch.cuda.empty_cache()

    C = 1 << chunk_log2
    rows_d = torch.empty((n_dp, C), dtype=torch.bfloat16, device=dev)
    rows_h = torch.empty((n_dp, C), dtype=torch.int16, pin_memory=True)
    slot = wf.view(torch.int16)[rank * S:(rank + 1) * S]
    compared = 0
    for c0 in range(0, S, C):
        n = min(C, S - c0)
        start = rank * S + c0

        def rows_of(t, n=n, start=start):
            for k in range(n_dp):
                synth.fill_device(rows_d[k, :n], d.kind, wl.seed,
                                  synth.tag(BUF_GRAD, cid, t, 0, k), start, d.eff_sigma, d.thr,
                                  d.outlier_mul)
            rows_h[:, :n].copy_(rows_d.view(torch.int16)[:, :n])
            return np.ascontiguousarray(rows_h[:, :n].numpy()).view(np.uint16).reshape(-1)

        w = synth.fill_host(F32, wl.seed, synth.tag(BUF_MASTER, cid), start, n, wl.master_sigma)
        m = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
        out = np.zeros(n, np.uint16)
        _oracle_steps(rows_of, ts, w, m, v, out, n_dp, wl)
        for name, got, want in (("master", W[c0:c0 + n], w), ("m", M[c0:c0 + n], m),
                                ("v", V[c0:c0 + n], v)):
            g = got.cpu().numpy()
            bad = np.count_nonzero(g.view(np.uint32) != want.view(np.uint32))
            assert bad == 0, f"{name}: {bad} of {n} elements at shard offset {c0} differ"
        g = slot[c0:c0 + n].cpu().numpy().view(np.uint16)
        bad = np.count_nonzero(g != out)
        assert bad == 0, f"weights: {bad} of {n} elements at shard offset {c0} differ"
        compared += n
        print(f"[full shard] config {cid}: {compared} of {S} elements bit-identical", flush=True)
    assert compared == S


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", [4, 7])
def test_every_element_of_the_accumulated_full_shard(cid):
    """Stage 2: 4 fp16 micro-batches reduced into the fp32 accumulator, then
    AdamW gated on the overflow flag; with cid 7 also the sum of squares on
    the last reduce, global-norm clipping (to a norm it must clip to) and
    the device-resident loss scale.  The oracle is given the device's sum of
    squares (its order differs by design); that sum is checked against the
    oracle's own within 1e-10."""
    wl = workload(cid)
    lay, _ = zs.zero_flatten_layout(wl.numels, wl.n_dp)
    S, n_dp, rank, micro = lay.shard, wl.n_dp, wl.rank, wl.micro_batches
    d = wl.grad
    ctl = wl.controls
    scale = 1.0 / (n_dp * wl.loss_scale * micro)
    print(f"\n[full shard] config {cid} rank {rank} S={S} n_dp={n_dp} micro={micro}", flush=True)
    dev = torch.device("cuda")
    slab = torch.empty((n_dp, S), dtype=torch.float16, device=dev)
    acc = torch.empty(S, dtype=torch.float32, device=dev)
    W = torch.empty(S, dtype=torch.float32, device=dev)
    synth.fill_device(W, F32, wl.seed, synth.tag(BUF_MASTER, cid), rank * S, wl.master_sigma)
    M = torch.zeros(S, dtype=torch.float32, device=dev)
    V = torch.zeros(S, dtype=torch.float32, device=dev)
    wf = torch.zeros(lay.n_pad, dtype=torch.bfloat16, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    ss = torch.zeros(1, dtype=torch.float64, device=dev)
    for mb in range(micro):
        for k in range(n_dp):
            synth.fill_device(slab[k], d.kind, wl.seed, synth.tag(BUF_GRAD, cid, 1, mb, k),
                              rank * S, d.eff_sigma, d.thr, d.outlier_mul)
        zs.zero_shard_reduce(slab, n_dp, S, S, acc, accumulate=mb > 0, overflow=flag,
                             sumsq=ss if ctl and mb == micro - 1 else None)
    if ctl:
        dls = zs.new_loss_scale(wl.loss_scale)
        torch.cuda.synchronize()
        d_ss = float(ss.item())
        s_ = 1.0 / (n_dp * micro) / wl.loss_scale
        max_norm = 0.5 * (d_ss ** 0.5) * s_
        assert oracle.clip_coef(d_ss, np.float32(s_), max_norm) < 1.0
        zs.zero_shard_adamw_ex(acc, W, M, V, wf, lay, rank,
                               zs.AdamWHParams(step=1, grad_scale=1.0 / (n_dp * micro), **wl.hp),
                               skip=flag, sumsq=ss, max_norm=max_norm, loss_scale=dls)
    else:
        zs.zero_shard_adamw(acc, W, M, V, wf, lay, rank,
                            zs.AdamWHParams(step=1, grad_scale=scale, **wl.hp), skip=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    del slab
    torch.cuda.empty_cache()

    C = 1 << 26
    rows_d = torch.empty((n_dp, C), dtype=torch.float16, device=dev)
    rows_h = torch.empty((n_dp, C), dtype=torch.int16, pin_memory=True)
    slot = wf.view(torch.int16)[rank * S:(rank + 1) * S]
    T = _threads()
    compared = 0
    o_ss_total = 0.0
    with ThreadPoolExecutor(max_workers=T) as pool:
        for c0 in range(0, S, C):
            n = min(C, S - c0)
            start = rank * S + c0
            cuts = [n * i // T for i in range(T + 1)]
            a = np.zeros(n, np.float32)
            o_flag = np.zeros((T, 1), np.uint32)
            o_ss = np.zeros((T, 1), np.float64)
            for mb in range(micro):
                for k in range(n_dp):
                    synth.fill_device(rows_d[k, :n], d.kind, wl.seed,
                                      synth.tag(BUF_GRAD, cid, 1, mb, k), start, d.eff_sigma,
                                      d.thr, d.outlier_mul)
                rows_h[:, :n].copy_(rows_d.view(torch.int16)[:, :n])
                flat = np.ascontiguousarray(rows_h[:, :n].numpy()).view(np.uint16).reshape(-1)
                last = mb == micro - 1

                def red(i, flat=flat, mb=mb, last=last):
                    lo, hi = cuts[i], cuts[i + 1]
                    oracle.reduce(flat[lo:], oracle.FP16, n_dp, n, hi - lo, a[lo:hi], mb > 0,
                                  overflow=o_flag[i], sumsq=o_ss[i] if ctl and last else None)
                list(pool.map(red, range(T)))
            assert not o_flag.any()
            o_ss_total += float(o_ss.sum())
            w = synth.fill_host(F32, wl.seed, synth.tag(BUF_MASTER, cid), start, n,
                                wl.master_sigma)
            m = np.zeros(n, np.float32)
            v = np.zeros(n, np.float32)
            out = np.zeros(n, np.uint16)

            def upd(i):
                lo, hi = cuts[i], cuts[i + 1]
                if ctl:
                    oracle.adamw_ex(a[lo:hi], w[lo:hi], m[lo:hi], v[lo:hi], out[lo:hi],
                                    oracle.BF16, hi - lo, 1, grad_scale=1.0 / (n_dp * micro),
                                    skip=o_flag[i], sumsq=np.array([d_ss]), max_norm=max_norm,
                                    loss_scale=np.array([wl.loss_scale], np.float32), **wl.hp)
                else:
                    oracle.adamw(a[lo:hi], w[lo:hi], m[lo:hi], v[lo:hi], out[lo:hi],
                                 oracle.BF16, hi - lo, 1, grad_scale=scale, skip=o_flag[i],
                                 **wl.hp)
            list(pool.map(upd, range(T)))
            for name, got, want in (("acc", acc[c0:c0 + n], a), ("master", W[c0:c0 + n], w),
                                    ("m", M[c0:c0 + n], m), ("v", V[c0:c0 + n], v)):
                g = got.cpu().numpy()
                bad = np.count_nonzero(g.view(np.uint32) != want.view(np.uint32))
                assert bad == 0, f"{name}: {bad} of {n} elements at shard offset {c0} differ"
            g = slot[c0:c0 + n].cpu().numpy().view(np.uint16)
            bad = np.count_nonzero(g != out)
            assert bad == 0, f"weights: {bad} of {n} elements at shard offset {c0} differ"
            compared += n
            print(f"[full shard] config {cid}: {compared} of {S} elements bit-identical", flush=True)
    assert compared == S
    if ctl:
        assert abs(d_ss - o_ss_total) <= 1e-10 * o_ss_total


@pytest.mark.timeout(900)
def test_every_element_of_the_dim0_fp32_row_shard():
    wl = workload(5)
    lay, _, _ = zs.zero_dim0_layout(wl.shapes, wl.n_dp)
    S, n_dp, rank = lay.shard, wl.n_dp, wl.rank
    d = wl.grad
    print(f"\n[full shard] config 5 rank {rank} S={S} n_dp={n_dp} steps={wl.steps}", flush=True)
    dev = torch.device("cuda")
    slab = torch.empty((n_dp, S), dtype=torch.float32, device=dev)
    W = torch.empty(S, dtype=torch.float32, device=dev)
    synth.fill_device(W, F32, wl.seed, synth.tag(BUF_MASTER, 5), rank * S, wl.master_sigma)
    M = torch.zeros(S, dtype=torch.float32, device=dev)
    V = torch.zeros(S, dtype=torch.float32, device=dev)
    wf = torch.zeros(lay.n_pad, dtype=torch.bfloat16, device=dev)
    for t in wl.steps:
        for k in range(n_dp):
            synth.fill_device(slab[k], F32, wl.seed, synth.tag(BUF_GRAD, 5, t, 0, k), rank * S,
                              d.eff_sigma, d.thr, d.outlier_mul)
        zs.zero_shard_step(slab, S, S, W, M, V, wf, lay, rank,
                           zs.AdamWHParams(step=t, grad_scale=1.0 / n_dp, **wl.hp))
    torch.cuda.synchronize()
    del slab
    torch.cuda.empty_cache()

    C = 1 << 25
    rows_d = torch.empty((n_dp, C), dtype=torch.float32, device=dev)
    rows_h = torch.empty((n_dp, C), dtype=torch.float32, pin_memory=True)
    slot = wf.view(torch.int16)[rank * S:(rank + 1) * S]
    T = _threads()
    compared = 0
    with ThreadPoolExecutor(max_workers=T) as pool:
        for c0 in range(0, S, C):
            n = min(C, S - c0)
            start = rank * S + c0
            cuts = [n * i // T for i in range(T + 1)]
            w = synth.fill_host(F32, wl.seed, synth.tag(BUF_MASTER, 5), start, n,
                                wl.master_sigma)
            m = np.zeros(n, np.float32)
            v = np.zeros(n, np.float32)
            out = np.zeros(n, np.uint16)
            for t in wl.steps:
                for k in range(n_dp):
                    synth.fill_device(rows_d[k, :n], F32, wl.seed, synth.tag(BUF_GRAD, 5, t, 0, k),
                                      start, d.eff_sigma, d.thr, d.outlier_mul)
                rows_h[:, :n].copy_(rows_d[:, :n])
                flat = np.ascontiguousarray(rows_h[:, :n].numpy()).reshape(-1)

                def run(i, flat=flat, t=t):
                    lo, hi = cuts[i], cuts[i + 1]
                    oracle.step(flat[lo:], oracle.FP32, n_dp, n, hi - lo, w[lo:hi], m[lo:hi],
                                v[lo:hi], out[lo:hi], oracle.BF16, t, grad_scale=1.0 / n_dp,
                                **wl.hp)
                list(pool.map(run, range(T)))
            for name, got, want in (("master", W[c0:c0 + n], w), ("m", M[c0:c0 + n], m),
                                    ("v", V[c0:c0 + n], v)):
                g = got.cpu().numpy()
                bad = np.count_nonzero(g.view(np.uint32) != want.view(np.uint32))
                assert bad == 0, f"{name}: {bad} of {n} elements at shard offset {c0} differ"
            g = slot[c0:c0 + n].cpu().numpy().view(np.uint16)
            bad = np.count_nonzero(g != out)
            assert bad == 0, f"weights: {bad} of {n} elements at shard offset {c0} differ"
            compared += n
            print(f"[full shard] config 5: {compared} of {S} elements bit-identical", flush=True)
    assert compared == S


def _same_f32(a, b):
    """bitwise, NaN matching NaN"""
    na, nb = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32))


@pytest.mark.timeout(900)
def test_every_element_of_the_8bit_shard():
    B = zs.ZERO_Q8_BLOCK
    wl = workload(6)
    lay, _ = zs.zero_flatten_layout(wl.numels, wl.n_dp, B)
    S, n_dp, rank = lay.shard, wl.n_dp, wl.rank
    nb = S // B
    d = wl.grad
    print(f"\n[full shard] config 6 rank {rank} S={S} n_dp={n_dp} steps={wl.steps}", flush=True)
    dev = torch.device("cuda")
    rows_q = torch.empty((n_dp, S), dtype=torch.int8, device=dev)
    rows_s = torch.empty((n_dp, nb), dtype=torch.float32, device=dev)
    tmp = torch.empty(S, dtype=torch.float32, device=dev)
    W = torch.empty(S, dtype=torch.float32, device=dev)
    synth.fill_device(W, F32, wl.seed, synth.tag(BUF_MASTER, 6), rank * S, wl.master_sigma)
    M = torch.zeros(S, dtype=torch.float32, device=dev)
    V = torch.zeros(S, dtype=torch.float32, device=dev)
    wq = torch.zeros(lay.n_pad, dtype=torch.int8, device=dev)
    wsc = torch.zeros(lay.n_pad // B, dtype=torch.float32, device=dev)
    for t in wl.steps:
        for k in range(n_dp):
            synth.fill_device(tmp, F32, wl.seed, synth.tag(BUF_GRAD, 6, t, 0, k), rank * S,
                              d.eff_sigma, d.thr, d.outlier_mul)
            zs.zero_q8_quantize(tmp, rows_q[k], rows_s[k])
        zs.zero_shard_step_q8(rows_q, rows_s, S, nb, S, W, M, V, wq, wsc, lay, rank,
                              zs.AdamWHParams(step=t, grad_scale=1.0 / n_dp, **wl.hp))
    torch.cuda.synchronize()
    del tmp
    torch.cuda.empty_cache()

    C = 1 << 25                                   # a whole number of blocks
    rows_d = torch.empty((n_dp, C), dtype=torch.float32, device=dev)
    rows_h = torch.empty((n_dp, C), dtype=torch.float32, pin_memory=True)
    T = _threads()
    compared = 0
    last = wl.steps[-1]
    with ThreadPoolExecutor(max_workers=T) as pool:
        for c0 in range(0, S, C):
            n = min(C, S - c0)
            nbk = n // B
            start = rank * S + c0
            blk_cuts = [nbk * i // T for i in range(T + 1)]
            w = synth.fill_host(F32, wl.seed, synth.tag(BUF_MASTER, 6), start, n,
                                wl.master_sigma)
            m = np.zeros(n, np.float32)
            v = np.zeros(n, np.float32)
            o_wq = np.zeros(n, np.int8)
            o_ws = np.zeros(nbk, np.float32)
            for t in wl.steps:
                for k in range(n_dp):
                    synth.fill_device(rows_d[k, :n], F32, wl.seed, synth.tag(BUF_GRAD, 6, t, 0, k),
                                      start, d.eff_sigma, d.thr, d.outlier_mul)
                rows_h[:, :n].copy_(rows_d[:, :n])
                x = np.ascontiguousarray(rows_h[:, :n].numpy())
                qs = list(pool.map(lambda k: oracle.q8_quantize(x[k], oracle.FP32), range(n_dp)))
                gq = np.concatenate([q for q, _ in qs])
                gs = np.concatenate([s_ for _, s_ in qs])
                if t == last:  # the device quantizer: every code and scale of the step's rows
                    for k in range(n_dp):
                        assert np.array_equal(rows_q[k, c0:c0 + n].cpu().numpy(), qs[k][0]), \
                            f"codes of row {k} at shard offset {c0}"
                        assert _same_f32(rows_s[k, c0 // B:c0 // B + nbk].cpu().numpy(), qs[k][1]), \
                            f"scales of row {k} at shard offset {c0}"

                def run(i, gq=gq, gs=gs, t=t):
                    b0, b1 = blk_cuts[i], blk_cuts[i + 1]
                    lo, hi = b0 * B, b1 * B
                    oracle.step_q8(gq[lo:], gs[b0:], n_dp, n, nbk, hi - lo, w[lo:hi], m[lo:hi],
                                   v[lo:hi], o_wq[lo:hi], o_ws[b0:b1], t, grad_scale=1.0 / n_dp,
                                   **wl.hp)
                list(pool.map(run, range(T)))
            for name, got, want in (("master", W[c0:c0 + n], w), ("m", M[c0:c0 + n], m),
                                    ("v", V[c0:c0 + n], v)):
                g = got.cpu().numpy()
                bad = np.count_nonzero(g.view(np.uint32) != want.view(np.uint32))
                assert bad == 0, f"{name}: {bad} of {n} elements at shard offset {c0} differ"
            lo = rank * S + c0
            assert np.array_equal(wq[lo:lo + n].cpu().numpy(), o_wq), f"weight codes at {c0}"
            assert _same_f32(wsc[lo // B:lo // B + nbk].cpu().numpy(), o_ws), f"weight scales at {c0}"
            compared += n
            print(f"[full shard] config 6: {compared} of {S} elements bit-identical", flush=True)
    assert compared == S
