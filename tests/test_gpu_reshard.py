"""GPU parity of the flat-range copies (through the C ABI) against the
oracle: gather (flatten, re-shard, consolidate), scatter (unflatten) and
re-shard ("ZeRO Optimizer, in depth", "Checkpoints: sharded on the way in,
consolidated on the way out").  The copies are bitwise, so every comparison
is exact, and guard bands around every destination show that nothing
outside it is written.  Pieces sit at random element offsets inside pooled
buffers, so every source/destination phase modulo 16 bytes occurs."""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_flatten_amd as zs
from synth import F32, tag
from synth.workloads import llama7b_numels

pytestmark = pytest.mark.gpu

NP = {2: np.uint16, 4: np.uint32}
TH = {2: torch.int16, 4: torch.int32}


def _dev(a, eb):
    return torch.from_numpy(a.view({2: np.int16, 4: np.int32}[eb]).copy()).cuda()


def _host(t, eb):
    return t.cpu().numpy().view(NP[eb])


def _place(rng, sizes, eb, slack=37):
    """Disjoint places for pieces of the given sizes in one pool (random
    element offsets, random gaps); returns the host pool and the offsets."""
    offs, cur = [], int(rng.integers(0, 9))
    for s in sizes:
        offs.append(cur)
        cur += s + int(rng.integers(0, slack))
    pool = rng.integers(0, 2 ** (8 * eb), size=cur + 16, dtype=np.uint64).astype(NP[eb])
    return pool, offs


def _cut(rng, n, max_pieces=14, holes=True):
    cuts = np.sort(rng.choice(np.arange(1, n), size=min(n - 1, max_pieces - 1), replace=False))
    b = [0] + [int(c) for c in cuts] + [n]
    spans = [(lo, hi - lo) for lo, hi in zip(b[:-1], b[1:])]
    if holes:
        spans = [s for s in spans if rng.random() > 0.2]
    rng.shuffle(spans)
    return spans  # (flat_off, len)


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("eb", [2, 4])
def test_gather_random_pieces(seed, eb):
    rng = np.random.default_rng(1000 * eb + seed)
    n = int(rng.integers(1, 40_000))
    spans = _cut(rng, max(n, 2))
    pool, offs = _place(rng, [ln for _, ln in spans], eb)
    dpool = _dev(pool, eb)
    pieces_d = [(dpool[o:o + ln], f) for (f, ln), o in zip(spans, offs)]
    pieces_h = [(pool[o:o + ln], f) for (f, ln), o in zip(spans, offs)]
    for begin, count in [(0, n), (int(rng.integers(0, n)), int(rng.integers(0, 9000))),
                         (max(0, n - 3000), 5000), (n + 17, 100)]:
        lead = int(rng.integers(0, 9))  # the destination's phase
        out_h = rng.integers(0, 2 ** (8 * eb), size=lead + count + 24, dtype=np.uint64).astype(NP[eb])
        out = _dev(out_h, eb)
        zs.zero_flat_gather(pieces_d, n, begin, out[lead:lead + count])
        got = _host(out, eb)
        want = out_h.copy()
        want[lead:lead + count] = oracle.flat_gather(pieces_h, n, begin, count) if pieces_h \
            else np.zeros(count, NP[eb])
        assert np.array_equal(got, want), (n, begin, count, lead)


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("eb", [2, 4])
def test_scatter_random_pieces(seed, eb):
    rng = np.random.default_rng(2000 * eb + seed)
    n = int(rng.integers(2, 40_000))
    spans = _cut(rng, n)
    pool, offs = _place(rng, [ln for _, ln in spans], eb)
    dpool = _dev(pool, eb)
    pieces_d = [(dpool[o:o + ln], f) for (f, ln), o in zip(spans, offs)]
    host_pool = pool.copy()
    pieces_h = [(host_pool[o:o + ln], f) for (f, ln), o in zip(spans, offs)]
    begin = int(rng.integers(0, n))
    count = int(rng.integers(0, n - begin + 1))
    lead = int(rng.integers(0, 9))
    src_h = rng.integers(0, 2 ** (8 * eb), size=lead + count, dtype=np.uint64).astype(NP[eb])
    src = _dev(src_h, eb)
    zs.zero_flat_scatter(src[lead:], begin, pieces_d)
    if pieces_h and count:
        oracle.flat_scatter(src_h[lead:], begin, pieces_h)
    assert np.array_equal(_host(dpool, eb), host_pool)  # pieces updated, gaps untouched


def _old_shards(flat, n_dp, align, fill_pad):
    _, n, n_pad, s = oracle.flatten_layout([flat.size], n_dp, align)
    padded = np.empty(n_pad, flat.dtype)
    padded[:n] = flat
    padded[n:] = fill_pad  # old padding that must not leak into the new shards
    return [padded[r * s:(r + 1) * s].copy() for r in range(n_dp)], s


@pytest.mark.parametrize("a,b,align", [(8, 16, 8), (8, 1, 8), (3, 5, 1), (64, 8, 8), (1, 64, 1),
                                       (16, 8, 8)])
@pytest.mark.parametrize("eb", [2, 4])
def test_reshard_matches_oracle(a, b, align, eb):
    n = 123_457
    rng = np.random.default_rng(a * 100 + b + eb)
    flat = rng.integers(1, 2 ** (8 * eb), size=n, dtype=np.uint64).astype(NP[eb])
    old, s_old = _old_shards(flat, a, align, fill_pad=NP[eb](0x5A5A))
    d_old = [_dev(x, eb) for x in old]
    _, _, _, s_new = oracle.flatten_layout([n], b, align)
    for r in range(b):
        out = torch.full((s_new + 8,), -1, dtype=TH[eb], device="cuda")
        zs.zero_reshard(d_old, n, r, out[:s_new])
        got = _host(out, eb)
        assert np.array_equal(got[:s_new], oracle.reshard(old, n, b, r, align)), f"rank {r}"
        assert np.all(got[s_new:] == NP[eb](2 ** (8 * eb) - 1))


def test_round_trip_8_to_16_to_8_on_device():
    n = 1_000_003
    flat = synth.fill_host(F32, 3, tag(5, 70), 0, n, 0.02)
    old, s8 = _old_shards(flat, 8, 8, fill_pad=np.float32(0))
    d8 = [torch.from_numpy(x).cuda() for x in old]
    _, _, _, s16 = oracle.flatten_layout([n], 16, 8)
    d16 = [torch.empty(s16, device="cuda") for _ in range(16)]
    for r in range(16):
        zs.zero_reshard(d8, n, r, d16[r])
    back = [torch.empty(s8, device="cuda") for _ in range(8)]
    for r in range(8):
        zs.zero_reshard(d16, n, r, back[r])
    for x, y in zip(old, back):
        assert np.array_equal(x.view(np.uint32), y.cpu().numpy().view(np.uint32))


def test_flatten_and_unflatten_a_model_on_device():
    """Per-tensor fp32 parameters (the GPT-2-like list of a small model) are
    flattened into 8 shards by gather and consolidated back by scatter."""
    numels = [50257 * 64, 64, 64, 1024 * 64 * 3, 3 * 64, 64 * 64, 64, 7, 4096 * 3 + 1, 11]
    offs, n, _, s = oracle.flatten_layout(numels, 8, 8)
    tensors = [synth.fill_host(F32, 4, tag(5, 71, i), 0, k, 0.02) for i, k in enumerate(numels)]
    d_t = [torch.from_numpy(t).cuda() for t in tensors]
    shards = [torch.empty(s, device="cuda") for _ in range(8)]
    for r in range(8):
        zs.zero_flat_gather(list(zip(d_t, offs)), n, r * s, shards[r])
    flat = np.concatenate(tensors)
    got = np.concatenate([x.cpu().numpy() for x in shards])
    assert np.array_equal(got[:n].view(np.uint32), flat.view(np.uint32))
    assert not np.any(got[n:])
    outs = [torch.full((k,), float("nan"), device="cuda") for k in numels]
    for r in range(8):
        zs.zero_flat_scatter(shards[r], r * s, list(zip(outs, offs)))
    for o, t in zip(outs, tensors):
        assert np.array_equal(o.cpu().numpy().view(np.uint32), t.view(np.uint32))


def test_many_pieces_span_several_launches():
    """More pieces than one launch's segment table holds (291 tensors of the
    7B list, scaled down), gathered into one shard."""
    numels = [max(1, k // 4096) for k in llama7b_numels()]
    assert len(numels) > 128
    offs, n, _, _ = oracle.flatten_layout(numels, 1, 1)
    rng = np.random.default_rng(11)
    pool, places = _place(rng, numels, 4, slack=5)
    dpool = _dev(pool, 4)
    pieces_d = [(dpool[p:p + k], int(f)) for k, p, f in zip(numels, places, offs)]
    pieces_h = [(pool[p:p + k], int(f)) for k, p, f in zip(numels, places, offs)]
    out = torch.empty(n + 5, dtype=torch.int32, device="cuda")
    zs.zero_flat_gather(pieces_d, n, 0, out)
    assert np.array_equal(_host(out, 4), oracle.flat_gather(pieces_h, n, 0, n + 5))


# ---- full size: the 7B model's fp32 master from 8 ranks to 16 ----------------

def _llama_layout(n_dp):
    lay, _ = zs.zero_flatten_layout(llama7b_numels(), n_dp, 8)
    return lay


def test_full_size_reshard_8_to_16_sampled():
    """Every old shard of the 7B fp32 master (8 ranks, 842M elements each) on
    the device.  New rank 5 of 16 spans old ranks 2 and 3; new rank 11 of 12
    ends in padding (12 does not divide N), which must read as zeros.  Checked
    at the old-shard boundaries, both ends and 2^20 random positions."""
    l8 = _llama_layout(8)
    n, s8 = l8.n, l8.shard
    tg = tag(5, 72)
    old = []
    for r in range(8):
        t = torch.empty(s8, device="cuda")
        synth.fill_device(t, F32, 6, tg, r * s8, 0.02)
        old.append(t)
    meta = [(r * s8, s8) for r in range(8)]
    rng = np.random.default_rng(12)
    for n_new, rank in ((16, 5), (12, 11)):
        s_new = _llama_layout(n_new).shard
        out = torch.empty(s_new, device="cuda")
        zs.zero_reshard(old, n, rank, out)
        torch.cuda.synchronize()
        lo = rank * s_new
        pos = np.concatenate([np.arange(4096), s_new - 4096 + np.arange(4096),
                              rng.integers(0, s_new, size=1 << 20)])
        for r in range(8):  # old boundaries inside this shard
            b = r * s8 - lo
            if 0 < b < s_new:
                pos = np.concatenate([pos, b - 64 + np.arange(128)])
        flat = lo + pos
        # the flat vector's element i is draw i of the stream (the old
        # shards were filled that way); the oracle's map names which old
        # shard holds it
        for i in flat[:: 1 << 14]:
            k, off = oracle.flat_locate(meta, n, int(i))
            assert (k, off) == ((int(i) // s8, int(i) % s8) if i < n else (-1, None))
        want = np.zeros(pos.size, np.float32)
        live = flat < n
        want[live] = synth.gather_host(F32, 6, tg, flat[live], 0.02)
        got = out[torch.from_numpy(pos).cuda()].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"{n_new} ranks, rank {rank}"
        if n_new == 12:
            assert lo + s_new > n and not np.any(got[~live]) and (~live).any()
        del out
    del old
    torch.cuda.empty_cache()


def test_full_size_conversions_every_element():
    """The 7B fp32 master in 8 old shards of 842M elements: re-sharded to new
    rank 5 of 16 and to new rank 11 of 12 (ending in padding), and
    consolidated into the model's 291 parameter tensors (one scatter per
    old shard).  A conversion moves each element of the flat vector, so the
    expected value of every element is the seeded stream's draw at its flat
    index (zero past N); it is drawn on the device by the generator's device
    build (bit-identical to its host build, tests/test_gpu_synth.py) and
    every element is compared bit for bit."""
    l8 = _llama_layout(8)
    n, s8 = l8.n, l8.shard
    tg = tag(5, 73)
    old = []
    for r in range(8):
        t = torch.empty(s8, device="cuda")
        synth.fill_device(t, F32, 7, tg, r * s8, 0.02)
        old.append(t)
    for n_new, rank in ((16, 5), (12, 11)):
        s_new = _llama_layout(n_new).shard
        print(f"\n[full] re-shard 8 -> {n_new}, rank {rank}, {s_new} elements", flush=True)
        out = torch.empty(s_new, device="cuda")
        zs.zero_reshard(old, n, rank, out)
        want = torch.zeros(s_new, device="cuda")
        lo = rank * s_new
        live = min(s_new, n - lo)
        synth.fill_device(want[:live], F32, 7, tg, lo, 0.02)
        assert torch.equal(out.view(torch.int32), want.view(torch.int32)), f"8 -> {n_new}"
        assert live < s_new or n_new == 16
        del out, want
    numels = llama7b_numels()
    _, offs = zs.zero_flatten_layout(numels, 8, 8)
    tensors = [torch.empty(k, device="cuda") for k in numels]
    pieces = list(zip(tensors, [int(o) for o in offs]))
    for r in range(8):
        zs.zero_flat_scatter(old[r], r * s8, pieces)
    del old
    torch.cuda.empty_cache()
    print(f"[full] consolidation into {len(numels)} tensors", flush=True)
    want = torch.empty(max(numels), device="cuda")
    for t, o in pieces:
        k = t.numel()
        synth.fill_device(want[:k], F32, 7, tg, o, 0.02)
        assert torch.equal(t.view(torch.int32), want[:k].view(torch.int32)), f"tensor at {o}"


def test_resume_on_another_gpu_count_keeps_the_trajectory():
    """3 steps on 4 ranks, the state (fp32 master, m, v and the bf16 weight
    buffer) converted on the device to 3 ranks, 3 more steps: bit-identical
    to the oracle's unsharded run over the same gradients (the average over
    4 ranks' rows, then over 3 ranks' rows)."""
    from tests.gpu_util import dev16, host_master, host_rows
    from synth import BF16
    from synth.workloads import GradDraw
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
    draw = GradDraw(BF16, 1e-3)
    n, cfg = 50_001, 122
    w = host_master(cfg, 0, n)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    wout = np.zeros(n, np.uint16)
    state, lay, wf = None, None, None
    for t in range(1, 7):
        n_dp = 4 if t <= 3 else 3
        new_lay, _ = zs.zero_flatten_layout([n], n_dp, 8)
        s = new_lay.shard
        if state is None:
            state = [[torch.from_numpy(host_master(cfg, r * s, s, pad_from=n)).cuda()
                      for r in range(n_dp)], [torch.zeros(s, device="cuda") for _ in range(n_dp)],
                     [torch.zeros(s, device="cuda") for _ in range(n_dp)]]
            wf = torch.zeros(new_lay.n_pad, dtype=torch.bfloat16, device="cuda")
        elif new_lay.n_dp != lay.n_dp:  # the GPU count changed: convert on the device
            conv = []
            for arr in state:
                out = [torch.empty(s, device="cuda") for _ in range(n_dp)]
                for r in range(n_dp):
                    zs.zero_reshard(arr, n, r, out[r])
                conv.append(out)
            state = conv
            wf_new = torch.empty(new_lay.n_pad, dtype=torch.bfloat16, device="cuda")
            zs.zero_flat_gather([(wf, 0)], n, 0, wf_new)
            wf = wf_new
        lay = new_lay
        for r in range(n_dp):
            rows = host_rows(cfg, t, 0, n_dp, r * s, s, draw, pad_from=n)
            zs.zero_shard_step(dev16(rows, zs.ZERO_BF16), s, s, state[0][r], state[1][r],
                               state[2][r], wf, lay, r,
                               zs.AdamWHParams(step=t, grad_scale=1.0 / n_dp, **hp))
        rows = host_rows(cfg, t, 0, n_dp, 0, n, draw)
        oracle.step(rows, oracle.BF16, n_dp, n, n, w, m, v, wout, oracle.BF16, t,
                    grad_scale=1.0 / n_dp, **hp)
    torch.cuda.synchronize()
    for arr, ref in zip(state, (w, m, v)):
        got = torch.cat(arr).cpu().numpy()[:n]
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    got_w = wf.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got_w[:n], wout) and not np.any(got_w[n:])
