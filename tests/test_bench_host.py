"""bench.py's host-side contract, on the CPU: one GPU only (more exits with
a message and a non-zero status before touching a device), the CPU
baselines' host description and thread count, and the all-core oracle
baseline equal, element for element, to one whole-range oracle call."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from synth import BF16, F32  # noqa: E402
from synth.synth_const import BUF_GRAD, BUF_MASTER  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_host_description_and_threads():
    d = bench.host_description()
    assert d.endswith(f"{os.cpu_count()} logical CPUs")
    assert 1 <= bench.host_threads() <= 16


def test_ranges_in_threads_equal_one_call():
    """The all-core baseline cuts the sample into contiguous ranges, one
    per thread; the oracle step is element-wise, so the ranges stepped in
    threads must equal one whole-range call bit for bit."""
    from concurrent.futures import ThreadPoolExecutor
    n, n_dp, T = 50_003, 8, 5
    hp = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
    rows = np.stack([synth.fill_host(BF16, 0, synth.tag(BUF_GRAD, 2, 1, 0, k), 0, n, 1e-3)
                     for k in range(n_dp)])
    flat = rows.reshape(-1)
    w0 = synth.fill_host(F32, 0, synth.tag(BUF_MASTER, 2), 0, n, 0.02)
    state = [w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)]
    ref = [w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)]
    cuts = [n * i // T for i in range(T + 1)]

    def run(i):
        a, b = cuts[i], cuts[i + 1]
        for t in (1, 2, 3):
            oracle.step(flat[a:], oracle.BF16, n_dp, n, b - a, state[0][a:b], state[1][a:b],
                        state[2][a:b], state[3][a:b], oracle.BF16, t, grad_scale=1.0 / n_dp, **hp)

    with ThreadPoolExecutor(max_workers=T) as pool:
        list(pool.map(run, range(T)))
    for t in (1, 2, 3):
        oracle.step(rows, oracle.BF16, n_dp, n, n, *ref, oracle.BF16, t, grad_scale=1.0 / n_dp, **hp)
    for got, want in zip(state, ref):
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


def test_roofline_and_ceiling_figures():
    """The bench line's kernel figures from given event times: achieved GB/s
    is the algorithmic bytes per launch over the average launch time, the
    ceiling is read at the step's own residency cap, and frac_of_ceiling is
    the ceiling's time over the step's."""
    S, n_dp = 1_000_000, 8
    r = dict(kms=[2.0, 2.0, 2.0], launch_bytes=42 * S, kernel="k", n_dp=n_dp,
             ceiling={5: 2.2, 7: 1.9, 10: 1.8})
    rl = bench.roofline_of(r, None)
    assert rl["launch_ms_avg"] == 2.0 and rl["achieved"] == 42 * S / 2e-3 / 1e9
    assert rl["frac"] == rl["achieved"] / bench.HBM_PEAK_GBPS
    ceil, frac = bench.ceiling_of(r)
    assert ceil["waves_per_cu"] == bench.STEP_CAPS[n_dp] == 7
    assert ceil["launch_ms_avg"] == 1.9 and frac == 1.9 / 2.0
    assert ceil["best_waves_per_cu"] == 10 and ceil["best_launch_ms_avg"] == 1.8
    assert bench.ceiling_of(dict(r, ceiling=None)) == (None, None)


def test_traffic_digest_covers_the_included_headers(tmp_path, monkeypatch):
    """A committed counter summary is used only while the kernel it measured
    is unchanged: the digest covers the kernel source and every header it
    includes, so an edit to a shared header also retires the summary."""
    csrc = "zero_sharded_mixed_flatten_amd/csrc/"
    assert bench.kernel_files(bench.KERNEL_SOURCE) == sorted(
        ["include/zero_shard.h", csrc + "host_common.h", csrc + "step_common.h",
         csrc + "zero_shard.hip"])
    assert csrc + "step_common.h" in bench.kernel_files(bench.Q8_SOURCE)
    assert csrc + "step_common.h" not in bench.kernel_files(bench.COPY_SOURCE)
    # a copy of the tree's sources with one header changed by one byte
    for rel in bench.kernel_files(bench.KERNEL_SOURCE):
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(bench.ROOT, rel), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = str(tmp_path / csrc / "zero_shard.hip")
    before = bench.source_digest(src)
    hdr = tmp_path / csrc / "step_common.h"
    hdr.write_bytes(hdr.read_bytes() + b"\n")
    assert bench.source_digest(src) != before
