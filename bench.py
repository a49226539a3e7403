#!/usr/bin/env python3
"""Benchmark: one data-parallel rank's sharded optimizer step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
reduce the n_dp ranks' 16-bit gradient rows for the owned shard, AdamW on
the fp32 master/m/v shard, cast into the shard's slot of the full 16-bit
weight buffer.  Default workload: the Llama-shaped 7B parameter list
(6,738,415,616 parameters) flattened over n_dp = 8 ranks, rank 1's shard of
842,301,952 parameters, bf16 gradients ~N(0, 1e-3) with 1% outliers x100,
fp32 master ~N(0, 0.02), AdamW lr 1e-4, betas (0.9, 0.999), eps 1e-8,
weight decay 0.1.  Inputs are drawn on the device and resident in HBM
before the timed region.

Prints one JSON line:
  value = params/s of the owned shard, with the algorithmic HBM GB/s and its
  fraction of 8 TB/s (bytes per parameter: 2 n_dp + 26 for the fused step),
  roofline = the dominant kernel's achieved GB/s from HIP events on the
  stream it runs on, traffic = counter-measured HBM bytes per launch when a
  counter summary for the current kernel source is committed under profiles/,
  cpu_baseline = the CPU oracle timed on a bounded sample on this host.
"""
import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "zero_sharded_mixed_flatten_amd", "csrc", "zero_shard.hip")
COPY_SOURCE = os.path.join(ROOT, "zero_sharded_mixed_flatten_amd", "csrc", "flat_copy.hip")
Q8_SOURCE = os.path.join(ROOT, "zero_sharded_mixed_flatten_amd", "csrc", "quant8.hip")
COUNTERS_DIR = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200,
                   help="timed steps (default 200: about a second of GPU time on the 7B shard)")
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", type=int, default=2,
                   help="workload: 1 GPT-2-XL n_dp=1, 2 7B n_dp=8 (default), "
                        "3 7B n_dp=64, 4 7B n_dp=8 fp16 with 4 micro-batches, "
                        "5 7B per-parameter dim-0 sharding n_dp=8 with fp32 gradients, "
                        "6 7B n_dp=8 with 8-bit blockwise rows and weights (ZeRO++), "
                        "7 configuration 4 with clipping and a dynamic loss scale")
    p.add_argument("--cpu-sample-log2", type=int, default=25,
                   help="CPU baseline sample: 2^k parameters of the shard")
    p.add_argument("--cpu-steps", type=int, default=12,
                   help="CPU baseline: optimizer steps over the sample (about 12 s single-threaded)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="time only the chosen workload (the plain default line also times "
                        "configurations 1, 3 and 4, the same-mix ceiling and the vendor copy)")
    p.add_argument("--bucket-elems", type=int, default=0, metavar="B",
                   help="single-launch 16-bit steps: issue the shard as consecutive buckets of B "
                        "elements, one library call each (0: one call for the whole shard)")
    p.add_argument("--graph", action="store_true",
                   help="single-launch 16-bit steps: capture the step (all its buckets) once as "
                        "a HIP graph that reads the step's constants from device memory, then "
                        "per step copy that step's constants and replay the graph")
    p.add_argument("--flags", action="store_true",
                   help="single-launch steps: also raise the overflow flag and sum the squares "
                        "of the scaled gradient (the shard's part of the global norm)")
    p.add_argument("--op", choices=["step", "reshard", "consolidate", "quantize", "dequantize"],
                   default="step",
                   help="step: the optimizer step (default); reshard: new rank 5 of 16's "
                        "shard of the 7B fp32 master, m and v from the 8-rank shards; "
                        "consolidate: the 8-rank fp32 master shards scattered into the "
                        "7B model's 291 per-parameter fp32 tensors; quantize / dequantize: "
                        "the 8-bit codec on rank 1's fp32 gradient of the 7B shard (to int8 "
                        "blocks, and back to bf16)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB (the known-size "
                        "reference that scales the HBM byte counters) --steps times and exit")
    return p.parse_args()


def calibrate_copy(mib, steps):
    """A plain copy kernel of known size: reads and writes mib MiB each."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": n,
                      "bytes_written_per_launch": n, "launches": steps}), flush=True)


def kernel_files(source=KERNEL_SOURCE):
    """The kernel source and every local header it includes, directly or
    through another header (quoted includes, looked up beside the source and
    in include/), sorted by path relative to the repository."""
    seen, todo = set(), [os.path.abspath(source)]
    dirs = [os.path.dirname(os.path.abspath(source)), os.path.join(ROOT, "include")]
    while todo:
        f = todo.pop()
        if f in seen:
            continue
        seen.add(f)
        for line in open(f, encoding="utf-8"):
            m = re.match(r'\s*#\s*include\s+"([^"]+)"', line)
            if m:
                for d in dirs:
                    h = os.path.join(d, m.group(1))
                    if os.path.exists(h):
                        todo.append(os.path.abspath(h))
                        break
    return sorted(os.path.relpath(f, ROOT) for f in seen)


def source_digest(source=KERNEL_SOURCE):
    """sha256 over the names and contents of kernel_files(source): a change
    to the kernel or to any header it includes changes the digest."""
    h = hashlib.sha256()
    for rel in kernel_files(source):
        data = open(os.path.join(ROOT, rel), "rb").read()
        h.update(f"{rel}\0{len(data)}\0".encode())
        h.update(data)
    return h.hexdigest()


def committed_traffic(workload_name, source=KERNEL_SOURCE):
    """Counter-measured HBM bytes per launch of the dominant kernel, from the
    committed counter summary -- only if it was taken on this kernel source
    and these headers (source_digest)."""
    path = os.path.join(COUNTERS_DIR, f"{workload_name}.counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != source_digest(source):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


STEP_CAPS = {1: 10, 8: 7, 64: 12}   # the fused 16-bit step's residency caps (waves per CU)
CEILING_CAPS = (5, 6, 7, 8, 10, 12, 16)


def _stream_mix():
    """libstream_mix.so: the same-mix ceiling kernel (calibration/)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "calibration", "libstream_mix.so"))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.stream_mix.argtypes = [vp, i32, i64, i64, vp, vp, vp, vp, i32, vp]
    lib.stream_mix.restype = ctypes.c_int
    return lib


def time_ceiling(slab, n_dp, S, master, m, v, slot, stream, caps, reps=10):
    """The same-mix ceiling on the step's own buffers: every byte the fused
    16-bit step moves, with its launch shape, and no arithmetic (the state
    is stored back as loaded).  Average kernel ms per cap (HIP events on the
    stream it runs on)."""
    import ctypes

    import torch
    lib = _stream_mix()
    out = {}
    for cap in caps:
        def call():
            rc = lib.stream_mix(slab.data_ptr(), n_dp, S, S, master.data_ptr(), m.data_ptr(),
                                v.data_ptr(), slot.data_ptr(), cap,
                                ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError("stream_mix refused its arguments")
        for _ in range(3):
            call()
        ev = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        out[cap] = statistics.fmean(a.elapsed_time(b) for a, b in ev)
    return out


def time_vendor_copy(nbytes, reps=10):
    """torch's device-to-device copy_ (HIP's own copy kernel) of nbytes:
    nbytes read and nbytes written per launch."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        dst.copy_(src)
    ev = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    ms = statistics.fmean(a.elapsed_time(b) for a, b in ev)
    del src, dst
    torch.cuda.empty_cache()
    gbps = 2 * nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "torch copy_ (device to device)", "bytes_read_per_launch": nbytes,
            "bytes_written_per_launch": nbytes, "launch_ms_avg": ms, "achieved": gbps,
            "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS}


def time_step_workload(config, steps, warmup, flags=False, bucket_elems=0, use_graph=False,
                       ceiling_caps=()):
    """Draw workload `config`'s inputs into HBM, run `warmup` untimed and
    `steps` timed steps of the hot path, and return the timings.  With
    ceiling_caps (single-launch 16-bit steps of 1, 8 or 64 rows), the
    same-mix ceiling is timed on the same buffers afterwards."""
    import torch

    import synth
    import zero_sharded_mixed_flatten_amd as zs
    from synth import F32
    from synth.synth_const import BUF_GRAD, BUF_MASTER
    from synth.workloads import workload

    dev = torch.device("cuda", 0)
    wl = workload(config)
    q8 = wl.comm == "q8"
    if wl.layout == "dim0":
        lay, _, _ = zs.zero_dim0_layout(wl.shapes, wl.n_dp)
    else:
        lay, _ = zs.zero_flatten_layout(wl.numels, wl.n_dp, zs.ZERO_Q8_BLOCK if q8 else 1)
    S, n_dp, rank = lay.shard, wl.n_dp, wl.rank
    draw = wl.grad
    gdt = {synth.BF16: zs.ZERO_BF16, synth.F16: zs.ZERO_FP16, synth.F32: zs.ZERO_FP32}[draw.kind]
    tdt = {zs.ZERO_BF16: torch.bfloat16, zs.ZERO_FP16: torch.float16,
           zs.ZERO_FP32: torch.float32}[gdt]
    gbytes = 4 if gdt == zs.ZERO_FP32 else 2
    micro = wl.micro_batches
    hp_kw = dict(wl.hp)

    # ---- inputs, resident in HBM -------------------------------------------
    nb = S // zs.ZERO_Q8_BLOCK
    slab_s = wfull_s = None
    if q8:
        # what each sender puts on the wire: its fp32 gradient for this shard,
        # quantized (before the timed region)
        slab = torch.empty((n_dp, S), dtype=torch.int8, device=dev)
        slab_s = torch.empty((n_dp, nb), dtype=torch.float32, device=dev)
        tmp = torch.empty(S, dtype=torch.float32, device=dev)
        for k in range(n_dp):
            synth.fill_device(tmp, draw.kind, wl.seed, synth.tag(BUF_GRAD, wl.cid, 1, 0, k),
                              rank * S, draw.eff_sigma, draw.thr, draw.outlier_mul)
            zs.zero_q8_quantize(tmp, slab[k], slab_s[k])
        del tmp
    else:
        slab = torch.empty((n_dp, S), dtype=tdt, device=dev)
        for k in range(n_dp):
            synth.fill_device(slab[k], draw.kind, wl.seed,
                              synth.tag(BUF_GRAD, wl.cid, 1, 0, k), rank * S,
                              draw.eff_sigma, draw.thr, draw.outlier_mul)
    master = torch.empty(S, dtype=torch.float32, device=dev)
    synth.fill_device(master, F32, wl.seed, synth.tag(BUF_MASTER, wl.cid), rank * S,
                      wl.master_sigma)
    m = torch.zeros(S, dtype=torch.float32, device=dev)
    v = torch.zeros(S, dtype=torch.float32, device=dev)
    if q8:
        wfull = torch.zeros(lay.n_pad, dtype=torch.int8, device=dev)
        wfull_s = torch.zeros(lay.n_pad // zs.ZERO_Q8_BLOCK, dtype=torch.float32, device=dev)
    else:
        wfull = torch.zeros(lay.n_pad, dtype=torch.bfloat16, device=dev)
    acc = torch.empty(S, dtype=torch.float32, device=dev) if micro > 1 else None
    flag = torch.zeros(1, dtype=torch.int32, device=dev) if micro > 1 or flags else None
    sumsq = loss_scale = None
    if wl.controls or flags:
        sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
    if wl.controls:
        loss_scale = zs.new_loss_scale(wl.loss_scale, dev)
    stream = torch.cuda.current_stream(dev)
    graph = None
    if use_graph:
        if micro != 1 or q8:
            print("--graph applies to the single-launch 16-bit steps", file=sys.stderr)
            sys.exit(2)
        # every step's constants in pinned host memory up front (no buffer is
        # rewritten while an earlier asynchronous copy may still read it), one
        # device buffer the captured kernels read
        host_consts = torch.empty((warmup + steps, 48), dtype=torch.uint8, pin_memory=True)
        for i in range(warmup + steps):
            hpi = zs.AdamWHParams(step=i + 1, grad_scale=1.0 / n_dp, **hp_kw)
            host_consts[i].copy_(torch.from_numpy(zs.zero_step_consts_make(hpi)))
        consts = zs.new_step_consts(dev)
        bucket = bucket_elems if bucket_elems > 0 else S
        fl = dict(overflow=flag, sumsq=sumsq) if flags else {}
        ws = (torch.empty(zs.zero_sumsq_workspace_bytes(bucket) // 8 + 1, dtype=torch.float64,
                          device=dev) if flags else None)

        def issue(st):
            if flags:
                flag.zero_()
                sumsq.zero_()
            for b0 in range(0, S, bucket):
                b1 = min(S, b0 + bucket)
                zs.zero_shard_step_dc(slab[:, b0:], S, b1 - b0, master[b0:], m[b0:], v[b0:],
                                      wfull, lay, rank, consts, shard_off=b0, stream=st,
                                      workspace=ws, **fl)

        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                issue(side)
        stream.wait_stream(side)
    torch.cuda.synchronize()

    # ---- one step of the hot path ------------------------------------------
    events = []

    def step(t, timed):
        if graph is not None:
            consts.copy_(host_consts[t - 1], non_blocking=True)
            e0 = torch.cuda.Event(enable_timing=True) if timed else None
            e1 = torch.cuda.Event(enable_timing=True) if timed else None
            if timed:
                e0.record(stream)
            graph.replay()
            if timed:
                e1.record(stream)
                events.append((e0, e1))
        elif micro == 1:
            hp = zs.AdamWHParams(step=t, grad_scale=1.0 / n_dp, **hp_kw)
            e0 = torch.cuda.Event(enable_timing=True) if timed else None
            e1 = torch.cuda.Event(enable_timing=True) if timed else None
            fl = dict(overflow=flag, sumsq=sumsq) if flags else {}
            if flags:  # caller-zeroed, outside the timed launch
                flag.zero_()
                sumsq.zero_()
            if timed:
                e0.record(stream)
            if q8:
                zs.zero_shard_step_q8(slab, slab_s, S, nb, S, master, m, v, wfull, wfull_s, lay,
                                      rank, hp, stream=stream, **fl)
            elif bucket_elems > 0:
                for b0 in range(0, S, bucket_elems):
                    b1 = min(S, b0 + bucket_elems)
                    zs.zero_shard_step(slab[:, b0:], S, b1 - b0, master[b0:], m[b0:], v[b0:],
                                       wfull, lay, rank, hp, shard_off=b0, stream=stream, **fl)
            else:
                zs.zero_shard_step(slab, S, S, master, m, v, wfull, lay, rank, hp, stream=stream,
                                   **fl)
            if timed:
                e1.record(stream)
                events.append((e0, e1))
        else:
            # stage-2 accumulation: one reduce per micro-batch (the same
            # resident slab stands in for each micro-batch's rows), then
            # AdamW gated on the overflow flag
            flag.zero_()
            if wl.controls:
                sumsq.zero_()
            for mb in range(micro):
                last = mb == micro - 1
                zs.zero_shard_reduce(slab, n_dp, S, S, acc, accumulate=mb > 0, overflow=flag,
                                     sumsq=sumsq if wl.controls and last else None,
                                     stream=stream)
            if wl.controls:
                # the loss scale lives on the device: grad_scale keeps the average only
                hp = zs.AdamWHParams(step=t, grad_scale=1.0 / (n_dp * micro), **hp_kw)
            else:
                hp = zs.AdamWHParams(step=t, grad_scale=1.0 / (n_dp * wl.loss_scale * micro),
                                     **hp_kw)
            e0 = torch.cuda.Event(enable_timing=True) if timed else None
            e1 = torch.cuda.Event(enable_timing=True) if timed else None
            if timed:
                e0.record(stream)
            if wl.controls:
                zs.zero_shard_adamw_ex(acc, master, m, v, wfull, lay, rank, hp, skip=flag,
                                       sumsq=sumsq, max_norm=1.0, loss_scale=loss_scale,
                                       stream=stream)
            else:
                zs.zero_shard_adamw(acc, master, m, v, wfull, lay, rank, hp, skip=flag,
                                    stream=stream)
            if timed:
                e1.record(stream)
                events.append((e0, e1))
            if wl.controls:
                zs.zero_loss_scale_update(loss_scale, flag, 2.0, 0.5, 2000, stream=stream)

    t = 0
    for _ in range(warmup):
        t += 1
        step(t, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        t += 1
        step(t, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    with_flags = " with the overflow flag and the sum of squares" if flags else ""
    if q8:
        bytes_per_param = n_dp * (1 + 4 / zs.ZERO_Q8_BLOCK) + 12 + 12 + 1 + 4 / zs.ZERO_Q8_BLOCK
        kernel = f"step_q8_kernel (fused dequantize + reduce + AdamW + quantize{with_flags})"
    elif micro == 1:
        bytes_per_param = gbytes * n_dp + 26
        kernel = f"step_quad_kernel (fused reduce + AdamW + cast{with_flags})"
        if use_graph:
            kernel += ", one graph replay per step, constants read from device memory"
    else:
        # 4 B written by the first reduce, 2 n_dp + 8 by each later one,
        # 30 by the gated AdamW (acc 4 + state 12 read, state 12 + weight 2 written)
        bytes_per_param = (gbytes * n_dp + 4) + (micro - 1) * (gbytes * n_dp + 8) + 30
        kernel = ("adamw_quad_kernel (gated AdamW with clipping and dynamic loss scale + cast; "
                  "timed launch)" if wl.controls else
                  "adamw_quad_kernel (gated AdamW + cast; timed launch)")
    kms = [a.elapsed_time(b) for a, b in events]
    r = dict(wl=wl, lay=lay, S=S, n_dp=n_dp, rank=rank, q8=q8, gdt=gdt, micro=micro,
             steps=steps, warmup=warmup, wall=wall, kms=kms, kernel=kernel,
             bytes_per_param=bytes_per_param, step_bytes=bytes_per_param * S,
             launch_bytes=bytes_per_param * S if micro == 1 else 30 * S, ceiling=None)
    if (ceiling_caps and micro == 1 and not q8 and gdt == zs.ZERO_BF16
            and n_dp in STEP_CAPS):
        r["ceiling"] = time_ceiling(slab, n_dp, S, master, m, v, wfull[rank * S:], stream,
                                    ceiling_caps)
    del slab, master, m, v, wfull, acc, slab_s, wfull_s
    torch.cuda.empty_cache()
    return r


def roofline_of(r, traffic):
    kms = r["kms"]
    k_avg = statistics.fmean(kms)
    achieved = r["launch_bytes"] / (k_avg * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": r["kernel"], "achieved": achieved,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic, "launch_ms_avg": k_avg, "launch_ms_min": min(kms),
            "launch_ms_median": statistics.median(kms),
            "algorithmic_bytes_per_launch": r["launch_bytes"]}


def ceiling_of(r):
    """The same-mix ceiling at the step's own residency cap and the best cap,
    and the step's kernel time as a fraction of the former."""
    c = r["ceiling"]
    if not c:
        return None, None
    own = STEP_CAPS[r["n_dp"]]
    best = min(c, key=c.get)
    k_avg = statistics.fmean(r["kms"])
    gb = lambda ms: r["launch_bytes"] / (ms * 1e-3) / 1e9
    return ({"kernel": "stream_mix (the step's bytes, launch shape and access, no arithmetic)",
             "waves_per_cu": own, "launch_ms_avg": c[own], "achieved": gb(c[own]),
             "unit": "GB/s", "frac": gb(c[own]) / HBM_PEAK_GBPS,
             "best_waves_per_cu": best, "best_launch_ms_avg": c[best],
             "best_frac": gb(c[best]) / HBM_PEAK_GBPS,
             "sweep_ms": {str(k): v for k, v in sorted(c.items())}},
            c[own] / k_avg)


def summary_of(r):
    """One workload's figures for the default line's other_configs."""
    rl = roofline_of(r, committed_traffic(r["wl"].name, Q8_SOURCE if r["q8"] else KERNEL_SOURCE))
    out = {"shard": r["S"], "n_dp": r["n_dp"], "rank": r["rank"],
           "bytes_per_param": r["bytes_per_param"], "steps": r["steps"],
           "warmup": r["warmup"], "ms_per_step": r["wall"] * 1e3 / r["steps"],
           "params_per_s": r["S"] * r["steps"] / r["wall"],
           "hbm_gbps": r["step_bytes"] * r["steps"] / r["wall"] / 1e9,
           "hbm_frac": r["step_bytes"] * r["steps"] / r["wall"] / 1e9 / HBM_PEAK_GBPS,
           "kernel": rl["kernel"], "kernel_ms_avg": rl["launch_ms_avg"],
           "kernel_gbps": rl["achieved"], "kernel_frac": rl["frac"],
           "algorithmic_bytes_per_launch": rl["algorithmic_bytes_per_launch"],
           "traffic": rl["traffic"]}
    if r["micro"] > 1:
        out["launches_per_step"] = r["micro"] + 1 + int(r["wl"].controls)
        out["kernel_bytes_per_param"] = 30
    ceil, frac = ceiling_of(r)
    if ceil:
        out["ceiling"] = ceil
        out["frac_of_ceiling"] = frac
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the sharded step is emulated with all n_dp "
              "ranks' gradient rows in one GPU's HBM, and no multi-GPU path is built. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, args.steps)
        return
    if args.op in ("quantize", "dequantize"):
        bench_codec(args)
        return
    if args.op != "step":
        bench_copies(args)
        return

    import torch

    import zero_sharded_mixed_flatten_amd as zs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    # the plain default line also times the other workloads, the same-mix
    # ceiling and the vendor copy
    plain = not (args.flags or args.graph or args.bucket_elems > 0 or args.no_extra)
    r = time_step_workload(args.config, args.steps, args.warmup, flags=args.flags,
                           bucket_elems=args.bucket_elems, use_graph=args.graph,
                           ceiling_caps=CEILING_CAPS if plain else ())
    wl, lay, S, n_dp, q8, micro = r["wl"], r["lay"], r["S"], r["n_dp"], r["q8"], r["micro"]
    wall, gdt = r["wall"], r["gdt"]
    # the committed counter summaries cover the variant without the flags
    # whose constants are kernel arguments (for the stage-2 workloads: the
    # timed AdamW launch)
    traffic = (committed_traffic(wl.name, Q8_SOURCE if q8 else KERNEL_SOURCE)
               if not args.flags and not args.graph else None)
    line = {
        "metric": "sharded AdamW step params/s and HBM GB/s (% of 8 TB/s), 7B n_dp=8 shard",
        "value": S * args.steps / wall,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "hbm_gbps": r["step_bytes"] / wall * args.steps / 1e9,
        "hbm_frac": r["step_bytes"] / wall * args.steps / 1e9 / HBM_PEAK_GBPS,
        "config": {"workload": wl.name, "n_params": lay.n, "n_dp": n_dp, "rank": r["rank"],
                   "shard": S, "layout": wl.layout,
                   "grad_dtype": "int8 blocks of 256 + fp32 scale" if q8 else
                   {zs.ZERO_BF16: "bf16", zs.ZERO_FP16: "fp16", zs.ZERO_FP32: "fp32"}[gdt],
                   "state_dtype": "fp32",
                   "weight_dtype": "int8 blocks of 256 + fp32 scale" if q8 else "bf16",
                   "micro_batches": micro, "bytes_per_param": r["bytes_per_param"],
                   "controls": "clip 1.0 + dynamic loss scale" if wl.controls else None,
                   "flags": "overflow + sum of squares" if args.flags and micro == 1 else None,
                   "bucket_elems": args.bucket_elems if args.bucket_elems > 0 and micro == 1
                   and not q8 else None,
                   "graph": "one captured graph, step constants in device memory"
                   if args.graph else None,
                   "launches_per_step": (-(-S // args.bucket_elems) if args.bucket_elems > 0
                                         and not q8 else 1) if micro == 1
                   else micro + 1 + int(wl.controls)},
        "roofline": roofline_of(r, traffic),
        "cpu_baseline": None,
    }
    ceil, frac = ceiling_of(r)
    if ceil:
        line["ceiling"] = ceil
        line["frac_of_ceiling"] = frac
    if plain:
        line["vendor_copy"] = time_vendor_copy(4 << 30)
        if args.config == 2:
            others = {}
            for c in (1, 3, 4):
                o = time_step_workload(c, min(args.steps, 10), min(args.warmup, 3),
                                       ceiling_caps=CEILING_CAPS)
                others[o["wl"].name] = summary_of(o)
            line["other_configs"] = others

    # ---- the oracle on the host: a reported baseline, never the target ------
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, S, r["rank"], args.cpu_sample_log2,
                                            args.cpu_steps)
        if micro == 1 and not q8:
            line["cpu_baseline_all_cores"] = cpu_baseline_all_cores(
                wl, S, r["rank"], args.cpu_sample_log2, 8 * args.cpu_steps)

    print(json.dumps(line), flush=True)


def bench_copies(args):
    """Checkpoint conversion on the device ("ZeRO Optimizer, in depth",
    "Checkpoints: sharded on the way in, consolidated on the way out"):
    bitwise copies, 8 bytes of HBM traffic per fp32 element (4 read, 4
    written).  A step converts one rank's worth of state."""
    import torch

    import synth
    import zero_sharded_mixed_flatten_amd as zs
    from synth import F32
    from synth.synth_const import BUF_M, BUF_MASTER, BUF_V
    from synth.workloads import llama7b_numels

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    numels = llama7b_numels()
    old, offs = zs.zero_flatten_layout(numels, 8, 8)
    n, s8 = old.n, old.shard
    stream = torch.cuda.current_stream(dev)
    events = []

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        return e0, e1

    if args.op == "reshard":
        new, _ = zs.zero_flatten_layout(numels, 16, 8)
        rank, s16 = 5, new.shard
        bufs = (BUF_MASTER, BUF_M, BUF_V)
        src = [[torch.empty(s8, device=dev) for _ in range(8)] for _ in bufs]
        for arr, b in zip(src, bufs):
            for r, t in enumerate(arr):
                synth.fill_device(t, F32, 1, synth.tag(b, 9), r * s8, 0.02)
        dst = [torch.empty(s16, device=dev) for _ in bufs]

        def step(record):
            for arr, d in zip(src, dst):
                call = lambda: zs.zero_reshard(arr, n, rank, d, stream=stream)
                if record:
                    events.append(timed(call))
                else:
                    call()
        elems_per_step, launches = 3 * s16, 3
        workload = "llama7b_fp32_state_reshard_8to16_rank5"
        metric = "re-shard of one rank's fp32 master, m and v, 7B model, 8 to 16 ranks"
        cfg = {"from_n_dp": 8, "to_n_dp": 16, "rank": rank, "arrays": 3, "shard": s16}
    else:
        src = [torch.empty(s8, device=dev) for _ in range(8)]
        for r, t in enumerate(src):
            synth.fill_device(t, F32, 1, synth.tag(BUF_MASTER, 9), r * s8, 0.02)
        tensors = [torch.empty(k, device=dev) for k in numels]
        pieces = list(zip(tensors, [int(o) for o in offs]))

        def step(record):
            for r in range(8):
                call = lambda: zs.zero_flat_scatter(src[r], r * s8, pieces, stream=stream)
                if record:
                    events.append(timed(call))
                else:
                    call()
        elems_per_step, launches = n, 8
        workload = "llama7b_fp32_master_consolidate_8"
        metric = "consolidation of the 7B fp32 master from 8 shards into per-parameter tensors"
        cfg = {"from_n_dp": 8, "tensors": len(numels), "n_params": n}
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = [a.elapsed_time(b) for a, b in events]
    launch_bytes = 8 * elems_per_step / launches
    k_avg = statistics.fmean(kms)
    achieved = launch_bytes / (k_avg * 1e-3) / 1e9
    line = {
        "metric": metric, "value": elems_per_step * args.steps / wall, "unit": "elements/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "hbm_gbps": 8 * elems_per_step * args.steps / wall / 1e9,
        "hbm_frac": 8 * elems_per_step * args.steps / wall / 1e9 / HBM_PEAK_GBPS,
        "config": dict(workload=workload, **cfg),
        "roofline": {"bound": "hbm", "kernel": "flat_copy_kernel", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": committed_traffic(workload, COPY_SOURCE), "launch_ms_avg": k_avg,
                     "launch_ms_min": min(kms), "algorithmic_bytes_per_launch": launch_bytes},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del src
        torch.cuda.empty_cache()
        line["cpu_baseline"] = cpu_baseline_copy(args.op, s8, n)
    print(json.dumps(line), flush=True)


def bench_codec(args):
    """The 8-bit blockwise codec of ZeRO++-style communication on the 7B
    shard (8 ranks, rank 1, 842,301,952 elements): quantize fp32 -> int8
    codes + fp32 block scales (4 bytes read, 1 + 4/256 written per element),
    or dequantize them to bf16 (1 + 4/256 read, 2 written)."""
    import numpy as np
    import torch

    import synth
    import zero_sharded_mixed_flatten_amd as zs
    from synth import F32
    from synth.synth_const import BUF_GRAD, outlier_threshold
    from synth.workloads import llama7b_numels

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    lay, _ = zs.zero_flatten_layout(llama7b_numels(), 8, zs.ZERO_Q8_BLOCK)
    S, rank = lay.shard, 1
    x = torch.empty(S, dtype=torch.float32, device=dev)
    synth.fill_device(x, F32, 0, synth.tag(BUF_GRAD, 6, 1, 0, 0), rank * S, 1e-3,
                      outlier_threshold(0.01), 100.0)
    q = torch.empty(S, dtype=torch.int8, device=dev)
    sc = torch.empty(zs.q8_blocks(S), dtype=torch.float32, device=dev)
    y = torch.empty(S, dtype=torch.bfloat16, device=dev)
    zs.zero_q8_quantize(x, q, sc)
    stream = torch.cuda.current_stream(dev)
    if args.op == "quantize":
        call = lambda: zs.zero_q8_quantize(x, q, sc, stream=stream)
        per_elem = 4 + 1 + 4 / zs.ZERO_Q8_BLOCK
        kernel = "q8_quantize_kernel"
    else:
        call = lambda: zs.zero_q8_dequantize(q, sc, y, stream=stream)
        per_elem = 1 + 4 / zs.ZERO_Q8_BLOCK + 2
        kernel = "q8_dequantize_pair_kernel"
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    events = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        events.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = [a.elapsed_time(b) for a, b in events]
    k_avg = statistics.fmean(kms)
    launch_bytes = per_elem * S
    achieved = launch_bytes / (k_avg * 1e-3) / 1e9
    line = {
        "metric": f"8-bit blockwise {args.op} of one rank's 7B gradient shard, elements/s",
        "value": S * args.steps / wall, "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "hbm_gbps": launch_bytes * args.steps / wall / 1e9,
        "hbm_frac": launch_bytes * args.steps / wall / 1e9 / HBM_PEAK_GBPS,
        "config": {"workload": f"llama7b_ndp8_q8_{args.op}", "elements": S,
                   "block": zs.ZERO_Q8_BLOCK, "bytes_per_element": per_elem},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": committed_traffic(f"llama7b_ndp8_q8_{args.op}", Q8_SOURCE),
                     "launch_ms_avg": k_avg, "launch_ms_min": min(kms),
                     "algorithmic_bytes_per_launch": launch_bytes},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        n = 1 << 22
        xs = synth.fill_host(F32, 0, synth.tag(BUF_GRAD, 6, 1, 0, 0), rank * S, n, 1e-3,
                             outlier_threshold(0.01), 100.0)
        qq, ss = oracle.q8_quantize(xs, oracle.FP32)
        t1 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t1 < 10.0:
            if args.op == "quantize":
                oracle.q8_quantize(xs, oracle.FP32)
            else:
                oracle.q8_dequantize(qq, ss, oracle.BF16)
            reps += 1
        dt = time.perf_counter() - t1
        line["cpu_baseline"] = {"value": reps * n / dt, "unit": "elements/s", "cores": 1,
                                "kind": "oracle", "host": host_description(),
                                "sample": f"the first {n} elements of the shard, {reps} calls, "
                                          f"single-threaded C oracle ({dt:.1f} s)"}
    print(json.dumps(line), flush=True)


def cpu_baseline_copy(op, s8, n):
    """The oracle's element-by-element copies on a bounded sample (about
    10 s, single-threaded).  reshard: new rank 5 of 16 built from 8 old
    shards of 2^24 elements (the sample's new shard straddles two old ones,
    as rank 5 of 16 does).  consolidate: the first 2^22 elements of old
    shard 0 scattered into the 7B model's 291 parameter tensors."""
    import numpy as np

    import oracle
    from synth.workloads import llama7b_numels
    t0 = time.perf_counter()
    reps = 0
    if op == "reshard":
        sample = 1 << 24
        per_call = sample // 2
        old = [np.full(sample, r, np.float32) for r in range(8)]
        while time.perf_counter() - t0 < 10.0:
            oracle.reshard(old, 8 * sample, 16, 5)
            reps += 1
        what = f"new rank 5 of 16 from 8 old shards of {sample} fp32 elements"
    else:
        per_call = 1 << 22
        numels = llama7b_numels()
        offs = np.concatenate([[0], np.cumsum(numels)[:-1]])
        keep = [i for i, o in enumerate(offs) if o < per_call]
        dests = [(np.zeros(numels[i], np.float32), int(offs[i])) for i in keep]
        src = np.ones(per_call, np.float32)
        while time.perf_counter() - t0 < 10.0:
            oracle.flat_scatter(src, 0, dests)
            reps += 1
        what = f"the first {per_call} elements of shard 0 into the parameter tensors they cover"
    dt = time.perf_counter() - t0
    return {"value": reps * per_call / dt, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "host": host_description(),
            "sample": f"{what} ({per_call} elements per call, {reps} calls, single-threaded C "
                      f"oracle, {dt:.1f} s)"}


def cpu_baseline(wl, S, rank, log2n, steps):
    import numpy as np

    import oracle
    import synth
    from synth import F32
    from synth.synth_const import BUF_GRAD, BUF_MASTER

    n = min(1 << log2n, S)
    draw = wl.grad
    rows = np.stack([synth.fill_host(draw.kind, wl.seed, synth.tag(BUF_GRAD, wl.cid, 1, 0, k),
                                     rank * S, n, draw.eff_sigma, draw.thr, draw.outlier_mul)
                     for k in range(wl.n_dp)])
    w = synth.fill_host(F32, wl.seed, synth.tag(BUF_MASTER, wl.cid), rank * S, n, wl.master_sigma)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    wout = np.zeros(n, np.uint16)
    acc = np.zeros(n, np.float32)
    gdt = {synth.BF16: oracle.BF16, synth.F16: oracle.FP16, synth.F32: oracle.FP32}[draw.kind]
    if wl.comm == "q8":
        qs = [oracle.q8_quantize(rows[k], oracle.FP32) for k in range(wl.n_dp)]
        gq = np.concatenate([q for q, _ in qs])
        gs = np.concatenate([s for _, s in qs])
        wq = np.zeros(n, np.int8)
        wsc = np.zeros(oracle.q8_blocks(n), np.float32)
        t0 = time.perf_counter()
        for t in range(1, steps + 1):
            oracle.step_q8(gq, gs, wl.n_dp, n, oracle.q8_blocks(n), n, w, m, v, wq, wsc, t,
                           grad_scale=1.0 / wl.n_dp, **wl.hp)
        dt = time.perf_counter() - t0
        return {"value": n * steps / dt, "unit": "params/s", "cores": 1, "kind": "oracle",
                "host": host_description(),
                "sample": f"first {n} parameters of rank {rank}'s shard, {wl.n_dp} 8-bit rows, "
                          f"{steps} optimizer steps, single-threaded C oracle ({dt:.1f} s)"}
    scale = np.array([wl.loss_scale], np.float32)
    good = np.zeros(1, np.int32)
    t0 = time.perf_counter()
    for t in range(1, steps + 1):
        if wl.micro_batches == 1:
            oracle.step(rows, gdt, wl.n_dp, n, n, w, m, v, wout, oracle.BF16, t,
                        grad_scale=1.0 / wl.n_dp, **wl.hp)
        else:
            flag = np.zeros(1, np.uint32)
            ss = np.zeros(1, np.float64)
            for mb in range(wl.micro_batches):
                last = mb == wl.micro_batches - 1
                oracle.reduce(rows, gdt, wl.n_dp, n, n, acc, mb > 0, overflow=flag,
                              sumsq=ss if wl.controls and last else None)
            if wl.controls:
                oracle.adamw_ex(acc, w, m, v, wout, oracle.BF16, n, t,
                                grad_scale=1.0 / (wl.n_dp * wl.micro_batches), skip=flag,
                                sumsq=ss, max_norm=1.0, loss_scale=scale, **wl.hp)
                oracle.loss_scale_update(scale, good, int(flag[0]), 2.0, 0.5, 2000)
            else:
                oracle.adamw(acc, w, m, v, wout, oracle.BF16, n, t,
                             grad_scale=1.0 / (wl.n_dp * wl.loss_scale * wl.micro_batches),
                             skip=flag, **wl.hp)
    dt = time.perf_counter() - t0
    return {"value": n * steps / dt, "unit": "params/s", "cores": 1, "kind": "oracle",
            "host": host_description(),
            "sample": f"first {n} parameters of rank {rank}'s shard, {wl.n_dp} gradient rows, "
                      f"{steps} optimizer steps, single-threaded C oracle ({dt:.1f} s)"}


def host_description():
    """The host the CPU baseline ran on: CPU model and logical CPU count."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {os.cpu_count()} logical CPUs"


def host_threads():
    """Worker threads for the all-core baseline: the cores this process may
    run on, at most 16 (one GPU's share of a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline_all_cores(wl, S, rank, log2n, steps):
    """The same single-threaded oracle step run on every host core at once:
    the sample is cut into one contiguous element range per thread and each
    thread steps its range (the update is element-wise, so the ranges are
    independent).  The oracle itself is unchanged; ctypes releases the GIL
    for the duration of each call."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import synth
    from synth import F32
    from synth.synth_const import BUF_GRAD, BUF_MASTER

    n = min(1 << log2n, S)
    draw = wl.grad
    rows = np.stack([synth.fill_host(draw.kind, wl.seed, synth.tag(BUF_GRAD, wl.cid, 1, 0, k),
                                     rank * S, n, draw.eff_sigma, draw.thr, draw.outlier_mul)
                     for k in range(wl.n_dp)])
    flat = rows.reshape(-1)
    w = synth.fill_host(F32, wl.seed, synth.tag(BUF_MASTER, wl.cid), rank * S, n, wl.master_sigma)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    wout = np.zeros(n, np.uint16)
    gdt = {synth.BF16: oracle.BF16, synth.F16: oracle.FP16, synth.F32: oracle.FP32}[draw.kind]
    threads = host_threads()
    cuts = [n * i // threads for i in range(threads + 1)]

    def run(i):
        a, b = cuts[i], cuts[i + 1]
        for t in range(1, steps + 1):
            # row k of the range starts at flat[a + k * n]
            oracle.step(flat[a:], gdt, wl.n_dp, n, b - a, w[a:b], m[a:b], v[a:b], wout[a:b],
                        oracle.BF16, t, grad_scale=1.0 / wl.n_dp, **wl.hp)

    with ThreadPoolExecutor(max_workers=threads) as pool:
        t0 = time.perf_counter()
        list(pool.map(run, range(threads)))
        dt = time.perf_counter() - t0
    return {"value": n * steps / dt, "unit": "params/s", "cores": threads, "kind": "oracle",
            "host": host_description(),
            "sample": f"first {n} parameters of rank {rank}'s shard, {wl.n_dp} gradient rows, "
                      f"{steps} optimizer steps, the single-threaded C oracle on {threads} "
                      f"contiguous ranges in {threads} threads ({dt:.1f} s)"}


if __name__ == "__main__":
    main()
