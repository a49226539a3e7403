"""The repository's host C/C++ code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): the oracle (oracle/oracle_zero.c),
the host input generator (synth/synth_cpu.c) and the library's host-only
layout code (layout.cpp: the flat and dim-0 layouts, segment maps, the
array_split pieces, the accounting), built by tests/sanitize/build.py.

Python is not built with ASan, so each check runs in a child process with
the ASan runtime preloaded; every finding is fatal there.  First the setup
is shown to bite (a planted heap overflow and a planted signed overflow in
a library built the same way are reported), then the oracle's pins run on
the sanitized oracle and generator, and the layout entry points are driven
through random and extreme arguments (sizes near 2^63, short output
arrays, null pointers) and compared with the sanitized oracle."""
import ctypes
import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

PINS = ["tests/test_oracle_accounting.py", "tests/test_oracle_adamw.py",
        "tests/test_oracle_control.py", "tests/test_oracle_convert.py",
        "tests/test_oracle_dim0.py", "tests/test_oracle_layout.py", "tests/test_oracle_q8.py",
        "tests/test_oracle_reduce.py", "tests/test_oracle_reshard.py", "tests/test_synth.py",
        "tests/test_q8_code_rule.py"]


def _asan_runtime():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def san():
    if _asan_runtime() is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_san_build", os.path.join(ROOT, "tests", "sanitize", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    oracle_so, synth_so, layout_so = mod.build()
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:"
                            "new_delete_type_mismatch=0:abort_on_error=0:exitcode=71",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=72",
               ORACLE_LIB=oracle_so, SYNTH_LIB=synth_so, ZERO_LAYOUT_SAN_LIB=layout_so)
    return dict(env=env, flags=mod.SAN)


def _run(env, args, timeout=900):
    return subprocess.run([sys.executable] + args, cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=timeout)


def _clean(r):
    out = r.stdout + r.stderr
    return (r.returncode == 0 and "ERROR: AddressSanitizer" not in out
            and "runtime error:" not in out), out[-4000:]


def test_the_sanitizers_catch_planted_mistakes(san):
    src = r"""
#include <stdint.h>
#include <stdlib.h>
int heap_overflow(int n) { int *a = malloc(n * sizeof(int)); a[n] = 1; int r = a[0]; free(a); return r; }
int64_t signed_overflow(int64_t a) { return a + INT64_MAX; }
"""
    with tempfile.TemporaryDirectory() as d:
        c, so = os.path.join(d, "planted.c"), os.path.join(d, "libplanted.so")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c11"] + san["flags"] + ["-o", so, c], check=True)
        r = _run(san["env"], ["-c", f"import ctypes; ctypes.CDLL({so!r}).heap_overflow(4)"])
        assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
        r = _run(san["env"], ["-c", "import ctypes; L = ctypes.CDLL(%r); "
                                    "L.signed_overflow.argtypes = [ctypes.c_int64]; "
                                    "L.signed_overflow(5)" % so])
        assert r.returncode != 0 and "signed integer overflow" in r.stderr


def test_the_oracle_pins_run_clean_under_the_sanitizers(san):
    """Every pin of the oracle and the generator, the sanitized builds in
    place of the regular ones (the converter tests' sweeps over all 2^32
    patterns are left to the regular run)."""
    r = _run(san["env"], ["-m", "pytest", "-q", "-p", "no:cacheprovider", "-x",
                          "-k", "not all_fp32_patterns"] + PINS)
    ok, out = _clean(r)
    assert ok, out
    assert " passed" in r.stdout


def test_the_host_layout_code_runs_clean_under_the_sanitizers(san):
    r = _run(san["env"], ["-c", "import tests.test_sanitizers as t; t.exercise_layout()"])
    ok, out = _clean(r)
    assert ok, out
    assert "layout calls:" in r.stdout


# ---------------------------------------------------------------------------
# driven in the sanitized child process (loads only the host-only layout
# library, not the GPU library)

class _Layout(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("n_pad", ctypes.c_int64), ("shard", ctypes.c_int64),
                ("align", ctypes.c_int64), ("n_dp", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class _Segment(ctypes.Structure):
    _fields_ = [("tensor", ctypes.c_int64), ("tensor_off", ctypes.c_int64),
                ("shard_off", ctypes.c_int64), ("len", ctypes.c_int64)]


def test_the_childs_structures_match_the_binding():
    import zero_sharded_mixed_flatten_amd as zs
    for mine, theirs in ((_Layout, zs.ZeroLayout), (_Segment, zs._Segment)):
        assert ctypes.sizeof(mine) == ctypes.sizeof(theirs)
        assert [(f[0], getattr(mine, f[0]).offset) for f in mine._fields_] == \
               [(f[0], getattr(theirs, f[0]).offset) for f in theirs._fields_]


def exercise_layout():
    import oracle
    L = ctypes.CDLL(os.environ["ZERO_LAYOUT_SAN_LIB"])
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lay_p = ctypes.POINTER(_Layout)
    L.zero_flatten_layout.argtypes = [vp, i64, i32, i64, vp, lay_p]
    L.zero_shard_segments.argtypes = [lay_p, vp, i64, i32, vp, i64, ctypes.POINTER(i64)]
    L.zero_dim0_layout.argtypes = [vp, vp, i64, i32, i64, vp, vp, lay_p]
    L.zero_dim0_segments.argtypes = [lay_p, vp, vp, i64, i32, vp, i64, ctypes.POINTER(i64)]
    L.zero_array_split_layout.argtypes = [i64, i32, vp, vp]
    L.zero_model_state_bytes.argtypes = [ctypes.c_double, ctypes.c_double, i32, ctypes.c_double,
                                         ctypes.POINTER(ctypes.c_double)]
    L.zero_comm_bytes.argtypes = [ctypes.c_double, ctypes.c_double, i32, ctypes.c_double,
                                  ctypes.c_double, ctypes.POINTER(ctypes.c_double)]
    L.zero_status_string.restype = ctypes.c_char_p
    ptr = lambda a: a.ctypes.data_as(vp) if a is not None else None
    rng = np.random.default_rng(5)
    big = np.iinfo(np.int64).max
    calls = 0

    def flatten(nums, n_dp, align, offs=True):
        nums = np.ascontiguousarray(nums, np.int64)
        o = np.zeros(max(1, nums.size), np.int64) if offs else None
        lay = _Layout()
        st = L.zero_flatten_layout(ptr(nums), nums.size, n_dp, align, ptr(o), ctypes.byref(lay))
        return st, lay, o

    def segments(lay, nums, rank, cap):
        nums = np.ascontiguousarray(nums, np.int64)
        out = (_Segment * max(1, cap))()
        cnt = i64(-1)
        st = L.zero_shard_segments(ctypes.byref(lay), ptr(nums), nums.size, rank, out, cap,
                                   ctypes.byref(cnt))
        return st, out, cnt.value

    for _ in range(400):
        k = int(rng.integers(0, 12))
        nums = rng.integers(0, 5000, size=k)
        n_dp = int(rng.integers(1, 70))
        align = int(rng.choice([1, 2, 8, 256, 4096]))
        st, lay, offs = flatten(nums, n_dp, align)
        calls += 1
        assert st == 0
        want = oracle.flatten_layout(nums, n_dp, align)
        assert (lay.n, lay.n_pad, lay.shard) == tuple(int(x) for x in want[1:])
        rank = int(rng.integers(0, n_dp))
        cap = int(rng.integers(0, k + 3))
        st, out, cnt = segments(lay, nums, rank, cap)
        calls += 1
        assert st == 0 and cnt >= 0
        q = oracle.shard_segments(nums, n_dp, rank, align)
        assert cnt == len(q)
        for j in range(min(cap, cnt)):
            assert (out[j].tensor, out[j].tensor_off, out[j].shard_off, out[j].len) == \
                   tuple(int(x) for x in q[j])
        starts = np.zeros(n_dp, np.int64)
        lens = np.zeros(n_dp, np.int64)
        n = int(nums.sum())
        assert L.zero_array_split_layout(n, n_dp, ptr(starts), ptr(lens)) == 0
        calls += 1
        assert starts.tolist() == [oracle.array_split_start(n, n_dp, r) for r in range(n_dp)]
        rows = rng.integers(0, 300, size=k)
        cols = rng.integers(0, 40, size=k)
        po, cr = np.zeros(max(1, k), np.int64), np.zeros(max(1, k), np.int64)
        dl = _Layout()
        st = L.zero_dim0_layout(ptr(np.ascontiguousarray(rows)), ptr(np.ascontiguousarray(cols)),
                                k, n_dp, align, ptr(po), ptr(cr), ctypes.byref(dl))
        calls += 1
        assert st == 0
        out = (_Segment * (2 * k + 2))()
        cnt = i64(-1)
        st = L.zero_dim0_segments(ctypes.byref(dl), ptr(np.ascontiguousarray(rows)),
                                  ptr(np.ascontiguousarray(cols)), k, rank, out, 2 * k + 2,
                                  ctypes.byref(cnt))
        calls += 1
        assert st == 0 and cnt.value <= 2 * k + 2
    # extreme sizes: rejected where a size would leave int64, exact where it fits
    for nums, n_dp, align in [([big], 1, 1), ([big, 1], 1, 1), ([big // 2, big // 2 + 1], 1, 1),
                              ([big // 2] * 2, 3, 1), ([big - 5], 4, 8), ([1 << 62], 2, 1 << 40),
                              ([1], 1 << 30, big // 4), ([0], 7, big), ([(1 << 62) + 3], 8, 1)]:
        st, lay, _ = flatten(nums, n_dp, align)
        calls += 1
        try:
            want = oracle.flatten_layout(nums, n_dp, align)
        except ValueError:
            want = None
        assert (st != 0) == (want is None), (nums, n_dp, align)
        if want is not None:
            assert (lay.n, lay.n_pad, lay.shard) == tuple(int(x) for x in want[1:])
            st, _, cnt = segments(lay, nums, n_dp - 1, 0)
            calls += 1
            assert st == 0 and cnt >= 1
    for rows, cols in [([big], [2]), ([1 << 40, 1 << 40], [1 << 22, 1 << 22]), ([3], [big])]:
        dl = _Layout()
        r_, c_ = np.array(rows, np.int64), np.array(cols, np.int64)
        st = L.zero_dim0_layout(ptr(r_), ptr(c_), r_.size, 8, 1, None, None, ctypes.byref(dl))
        calls += 1
        assert st != 0
    # null pointers and bad sizes: a status, never a crash
    lay = _Layout()
    assert L.zero_flatten_layout(None, 3, 4, 1, None, ctypes.byref(lay)) != 0
    assert L.zero_flatten_layout(None, 0, 4, 1, None, None) != 0
    assert L.zero_array_split_layout(10, 0, None, None) != 0
    assert L.zero_shard_segments(None, None, 0, 0, None, 0, None) != 0
    res = ctypes.c_double()
    for stage in range(-1, 5):
        L.zero_model_state_bytes(7e9, 8, stage, 12, ctypes.byref(res))
        L.zero_comm_bytes(7e9, 8, stage, 2, 2, ctypes.byref(res))
        calls += 2
    for s in range(-2, 8):
        assert L.zero_status_string(s)
    print(f"layout calls: {calls}", flush=True)
