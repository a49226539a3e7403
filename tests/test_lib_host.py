"""The C-ABI library on the CPU: it loads, exports every entry point the
header declares, and its host-only parts (layout, segments, accounting,
argument validation) agree with the oracle.  No kernel is launched here."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle
import zero_sharded_mixed_flatten_amd as zs
from synth.workloads import gpt2xl_numels, llama7b_numels

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zero_shard.h")
GOLD = os.path.join(ROOT, "tests", "golden")


def _declared():
    src = open(HEADER).read()
    return re.findall(r"^ZERO_API\s+[\w\s\*]*?\b(zero_\w+)\s*\(", src, flags=re.M)


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) == 28, names
    lib = ctypes.CDLL(zs.library_path())
    for n in names:
        assert hasattr(lib, n), n
    assert lib.zero_abi_version() == zs.ABI_VERSION


def test_one_hip_runtime_whatever_the_import_order():
    """torch ships its own HIP runtime; the package must bind to it even
    when imported before torch, or the process holds two runtimes and
    torch's streams are not valid in the library's (launches fail).  A
    fresh process imports the package first, then torch, and must map one
    libamdhip64 only."""
    import subprocess
    import sys
    code = ("import zero_sharded_mixed_flatten_amd, torch; "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'amdhip64' in l}))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    maps = eval(r.stdout.strip().splitlines()[-1])
    assert len(maps) == 1, maps


def test_status_strings():
    lib = ctypes.CDLL(zs.library_path())
    lib.zero_status_string.restype = ctypes.c_char_p
    for code in range(5):
        assert lib.zero_status_string(code).startswith(b"ZERO_")
    assert lib.zero_status_string(99) == b"unknown zero_status"


def test_tiny_layout_golden():
    g = json.load(open(os.path.join(GOLD, "tiny_layout.json")))
    lay, offs = zs.zero_flatten_layout(g["numels"], g["n_dp"], g["align"])
    assert (lay.n, lay.n_pad, lay.shard, lay.n_dp) == (g["n"], g["n_pad"], g["shard"], g["n_dp"])
    assert zs.zero_shard_segments(lay, g["numels"], g["rank"]) == \
        [(0, g["slot_begin"], 0, g["slot_end"] - g["slot_begin"])]


@pytest.mark.parametrize("seed", range(30))
def test_layout_and_segments_match_oracle(seed):
    rng = np.random.default_rng(seed)
    numels = [int(x) for x in rng.integers(0, 300, size=int(rng.integers(0, 12)))]
    n_dp = int(rng.integers(1, 70))
    align = int(rng.choice([1, 2, 8, 64]))
    lay, offs = zs.zero_flatten_layout(numels, n_dp, align)
    o_offs, n, n_pad, s = oracle.flatten_layout(numels, n_dp, align)
    assert (lay.n, lay.n_pad, lay.shard) == (n, n_pad, s)
    assert np.array_equal(offs, o_offs)
    for r in sorted({0, n_dp - 1, int(rng.integers(0, n_dp))}):
        assert zs.zero_shard_segments(lay, numels, r) == oracle.shard_segments(numels, n_dp, r, align)


@pytest.mark.parametrize("numels,n_dp", [(llama7b_numels(), 8), (llama7b_numels(), 64),
                                         (gpt2xl_numels(), 1)])
def test_model_layouts_match_oracle(numels, n_dp):
    lay, offs = zs.zero_flatten_layout(numels, n_dp)
    o = oracle.flatten_layout(numels, n_dp)
    assert (lay.n, lay.n_pad, lay.shard) == o[1:] and np.array_equal(offs, o[0])
    for r in sorted({0, min(1, n_dp - 1), n_dp - 1}):
        assert zs.zero_shard_segments(lay, numels, r) == oracle.shard_segments(numels, n_dp, r)


@pytest.mark.parametrize("args", [([4], 0, 1), ([4], 2, 0), ([-1], 2, 1),
                                  ([2 ** 62, 2 ** 62], 1, 1), ([2 ** 62 + 1], 2, 2 ** 61)])
def test_layout_rejects_invalid(args):
    with pytest.raises(zs.ZeroError) as e:
        zs.zero_flatten_layout(*args)
    assert e.value.status == zs.ZERO_EINVAL


def test_segments_reject_inconsistent_numels():
    lay, _ = zs.zero_flatten_layout([10, 20], 4)
    with pytest.raises(zs.ZeroError):
        zs.zero_shard_segments(lay, [10, 21], 0)
    with pytest.raises(zs.ZeroError):
        zs.zero_shard_segments(lay, [10, 20], 4)


def test_accounting_matches_oracle_and_pages():
    g = json.load(open(os.path.join(GOLD, "accounting.json")))
    for e in g["state_memory"]:
        got = zs.zero_model_state_bytes(e["n"], e["n_dp"], e["stage"], 12)
        assert got == oracle.model_state_bytes(e["n"], e["n_dp"], e["stage"], 12)
        assert abs(got / 1e9 - e["gb"]) <= e["abs_tol_gb"]
    for e in g["comm"]:
        got = zs.zero_comm_bytes(e["n"], e["n_dp"], e["stage"], e["param_bytes"], e["grad_bytes"])
        assert abs(got / 1e9 - e["gb"]) <= e["abs_tol_gb"]
    for stage in range(4):
        for n_dp in (1, 3, 8, 64):
            assert zs.zero_comm_bytes(1e9, n_dp, stage) == pytest.approx(
                oracle.comm_bytes(1e9, n_dp, stage), rel=1e-15)
    with pytest.raises(zs.ZeroError):
        zs.zero_model_state_bytes(1e9, 8, 4)


# ---------------------------------------------------------------------------
# argument validation of the device entry points: every case here must be
# rejected on the host before any launch, so it is exercised with made-up
# addresses -- and therefore only where no GPU is visible.

HIP_ERROR_NO_DEVICE = 100


def _no_gpu():
    """True only when no GPU can be reached; any doubt counts as a GPU.
    No GPU device node (/dev/kfd, /dev/dri), the HIP runtime that the
    library binds to (the process's libamdhip64, loaded with torch) reports
    no device, and torch sees none."""
    if os.path.exists("/dev/kfd") or os.path.exists("/dev/dri"):
        return False
    try:
        import torch
        if torch.cuda.device_count() != 0:
            return False
        hip = ctypes.CDLL("libamdhip64.so.7")
        n = ctypes.c_int(-1)
        rc = hip.hipGetDeviceCount(ctypes.byref(n))
        return rc == HIP_ERROR_NO_DEVICE or (rc == 0 and n.value == 0)
    except Exception:
        return False


cpu_only = pytest.mark.skipif(not _no_gpu(), reason="uses made-up device addresses")

L = zs._lib
P = ctypes.c_void_p
BASE = 1 << 40


def _hp(**kw):
    h = zs.AdamWHParams(**kw)
    return h._c()


def _step(grads=BASE, ld=1024, length=1024, master=BASE + (1 << 30), m=BASE + (2 << 30),
          v=BASE + (3 << 30), wfull=BASE + (4 << 30), lay=None, rank=1, shard_off=0,
          hp=None, ovf=None, ssq=None, gdt=0, wdt=0, ws=None, ws_bytes=None):
    if lay is None:
        lay = zs.zero_flatten_layout([4096], 4)[0]
    hp = hp or _hp()
    if ssq and ws is None:
        ws = BASE + (5 << 30)
    if ws_bytes is None:
        ws_bytes = zs.zero_sumsq_workspace_bytes(max(length, 0)) if ws else 0
    return L.zero_shard_step(P(grads), gdt, ld, length, P(master), P(m), P(v), P(wfull), wdt,
                             ctypes.byref(lay), rank, shard_off, ctypes.byref(hp),
                             P(ovf) if ovf else None, P(ssq) if ssq else None,
                             P(ws) if ws else None, ws_bytes, None)


@cpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(rank=4), zs.ZERO_EINVAL), (dict(rank=-1), zs.ZERO_EINVAL),
    (dict(ld=1000), zs.ZERO_EINVAL), (dict(length=-1), zs.ZERO_EINVAL),
    (dict(gdt=3), zs.ZERO_EINVAL), (dict(wdt=5), zs.ZERO_EINVAL),
    (dict(grads=0), zs.ZERO_EINVAL), (dict(master=0), zs.ZERO_EINVAL),
    (dict(hp=_hp(step=0)), zs.ZERO_EINVAL), (dict(hp=_hp(beta1=1.0)), zs.ZERO_EINVAL),
    (dict(hp=_hp(beta2=-0.1)), zs.ZERO_EINVAL), (dict(hp=_hp(eps=0.0)), zs.ZERO_EINVAL),
    (dict(hp=_hp(grad_scale=float("inf"))), zs.ZERO_EINVAL),
    (dict(hp=_hp(lr=float("nan"))), zs.ZERO_EINVAL),
    (dict(hp=_hp(weight_decay=-1.0)), zs.ZERO_EINVAL),
    (dict(shard_off=1, length=1024), zs.ZERO_ERANGE),
    (dict(shard_off=-1), zs.ZERO_EINVAL),
    (dict(length=1025, ld=1025), zs.ZERO_ERANGE),
    # rows spanning more than 2^60 elements: byte offsets would leave int64
    (dict(ld=1 << 61), zs.ZERO_EINVAL),
    (dict(ld=(1 << 60) // 3), zs.ZERO_EINVAL),
    (dict(m=BASE + (1 << 30) + 4092), zs.ZERO_EALIAS),       # m overlaps master's tail
    (dict(v=BASE + 2046), zs.ZERO_EALIAS),                    # v inside row 0
    (dict(master=BASE + 3 * 1024 * 2), zs.ZERO_EALIAS),       # master on the last row
    (dict(wfull=BASE + (3 << 30) - 2 * 1024), zs.ZERO_EALIAS),  # slot over v
    (dict(ovf=BASE + 100), zs.ZERO_EALIAS),
    (dict(ssq=BASE + (2 << 30) + 8), zs.ZERO_EALIAS),
    # the sum of squares' workspace: required, 8-byte aligned, large enough, disjoint
    (dict(ssq=BASE + (6 << 30), ws=0), zs.ZERO_EINVAL),
    (dict(ssq=BASE + (6 << 30), ws=BASE + (5 << 30) + 4), zs.ZERO_EINVAL),
    (dict(ssq=BASE + (6 << 30), ws_bytes=zs.zero_sumsq_workspace_bytes(1024) - 1),
     zs.ZERO_EINVAL),
    (dict(ssq=BASE + (6 << 30), ws=BASE + (3 << 30)), zs.ZERO_EALIAS),      # over v
    (dict(ssq=BASE + (5 << 30) + 64), zs.ZERO_EALIAS),                      # sumsq inside it
])
def test_step_rejects_bad_arguments(kw, status):
    assert _step(**kw) == status


@cpu_only
def test_step_bad_layout_and_empty_range():
    lay = zs.zero_flatten_layout([4096], 4)[0]
    bad = zs.ZeroLayout(lay.n, lay.n_pad + 1, lay.shard, lay.align, lay.n_dp, 0)
    assert _step(lay=bad) == zs.ZERO_EINVAL
    # a consistent layout whose buffer spans more than 2^60 elements
    huge = zs.ZeroLayout(1 << 61, 1 << 61, 1 << 58, 1, 8, 0)
    assert _step(lay=huge) == zs.ZERO_EINVAL
    # an empty range is a no-op that needs no buffers at all
    assert _step(length=0, grads=0, master=0, m=0, v=0, wfull=0) == zs.ZERO_OK


@cpu_only
def test_reduce_and_adamw_reject_bad_arguments():
    R = L.zero_shard_reduce
    assert R(P(BASE), 0, 0, 16, 16, P(BASE + 4096), 0, None, None, None, 0,
             None) == zs.ZERO_EINVAL
    assert R(P(BASE), 0, 2, 8, 16, P(BASE + 4096), 0, None, None, None, 0,
             None) == zs.ZERO_EINVAL
    assert R(P(BASE), 3, 2, 16, 16, P(BASE + 4096), 0, None, None, None, 0,
             None) == zs.ZERO_EINVAL
    assert R(P(BASE), 0, 2, 16, 16, P(BASE + 40), 0, None, None, None, 0,
             None) == zs.ZERO_EALIAS
    assert R(P(BASE), 0, 2, 1 << 62, 16, P(BASE + 4096), 0, None, None, None, 0,
             None) == zs.ZERO_EINVAL                                      # rows past 2^60
    assert R(P(BASE), 0, 2, 16, 16, P(BASE + 4096), 0, P(BASE + 4096 + 60), None,
             None, 0, None) == zs.ZERO_EALIAS
    assert R(None, 0, 2, 16, 0, None, 0, None, None, None, 0, None) == zs.ZERO_OK
    wsb = zs.zero_sumsq_workspace_bytes(16)
    ssq, ws = P(BASE + 8192), P(BASE + 16384)
    assert R(P(BASE), 0, 2, 16, 16, P(BASE + 4096), 0, None, ssq, None, 0,
             None) == zs.ZERO_EINVAL                                      # no workspace
    assert R(P(BASE), 0, 2, 16, 16, P(BASE + 4096), 0, None, ssq, ws, wsb - 8,
             None) == zs.ZERO_EINVAL                                      # too small
    assert R(P(BASE), 0, 2, 16, 16, P(BASE + 4096), 0, None, ssq, P(BASE + 4000), wsb,
             None) == zs.ZERO_EALIAS                                      # over acc
    assert zs.zero_sumsq_workspace_bytes(0) == 8 * (256 + 4096)
    assert zs.zero_sumsq_workspace_bytes(257) == 8 * (256 + 2 + 4096)
    with pytest.raises(ValueError):
        zs.zero_sumsq_workspace_bytes(-1)
    A = L.zero_shard_adamw
    lay = zs.zero_flatten_layout([4096], 4)[0]
    hp = _hp()
    args = [P(BASE), P(BASE + (1 << 30)), P(BASE + (2 << 30)), P(BASE + (3 << 30)),
            P(BASE + (4 << 30)), 0, ctypes.byref(lay), 1, 0, 1024, ctypes.byref(hp),
            None, None]
    bad = list(args)
    bad[8], bad[9] = 512, 1024
    assert A(*bad) == zs.ZERO_ERANGE
    bad = list(args)
    bad[11] = P(BASE + (1 << 30) + 16)  # skip flag inside master
    assert A(*bad) == zs.ZERO_EALIAS
    bad = list(args)
    bad[1] = P(BASE + 4000)  # master over acc
    assert A(*bad) == zs.ZERO_EALIAS


@cpu_only
def test_controls_reject_bad_arguments():
    U = L.zero_loss_scale_update
    assert U(None, P(BASE + 64), 2.0, 0.5, 10, None) == zs.ZERO_EINVAL
    assert U(P(BASE), None, 2.0, 0.5, 10, None) == zs.ZERO_EINVAL
    assert U(P(BASE), P(BASE + 64), 0.5, 0.5, 10, None) == zs.ZERO_EINVAL      # growth < 1
    assert U(P(BASE), P(BASE + 64), float("inf"), 0.5, 10, None) == zs.ZERO_EINVAL
    assert U(P(BASE), P(BASE + 64), 2.0, 0.0, 10, None) == zs.ZERO_EINVAL      # backoff <= 0
    assert U(P(BASE), P(BASE + 64), 2.0, 1.5, 10, None) == zs.ZERO_EINVAL      # backoff > 1
    assert U(P(BASE), P(BASE + 64), 2.0, 0.5, 0, None) == zs.ZERO_EINVAL       # interval < 1
    assert U(P(BASE), P(BASE + 4), 2.0, 0.5, 10, None) == zs.ZERO_EALIAS       # flag inside state
    A = L.zero_shard_adamw_ex
    lay = zs.zero_flatten_layout([4096], 4)[0]
    hp = _hp()
    base = [P(BASE), P(BASE + (1 << 30)), P(BASE + (2 << 30)), P(BASE + (3 << 30)),
            P(BASE + (4 << 30)), 0, ctypes.byref(lay), 1, 0, 1024, ctypes.byref(hp)]
    ctl = zs._StepControl(None, P(BASE + (1 << 30) + 8).value, 1.0, None)  # sumsq inside master
    assert A(*base, ctypes.byref(ctl), None) == zs.ZERO_EALIAS
    ctl = zs._StepControl(None, None, float("nan"), None)
    assert A(*base, ctypes.byref(ctl), None) == zs.ZERO_EINVAL
    ctl = zs._StepControl(None, None, 0.0, P(BASE + (2 << 30) + 100).value)  # loss scale inside m
    assert A(*base, ctypes.byref(ctl), None) == zs.ZERO_EALIAS


@pytest.mark.parametrize("step", [1, 2, 7, 1000])
@pytest.mark.parametrize("grad_scale", [1.0 / 8, 1.0 / 3])
def test_step_consts_equal_the_oracles(step, grad_scale):
    """zero_step_consts_make forms the ten constants by the same rule as the
    oracle (separate code, same stated rounding): equal bit for bit, with
    grad_scale kept as the double it was given."""
    hp = zs.AdamWHParams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1,
                         grad_scale=grad_scale, step=step)
    got = zs.zero_step_consts_make(hp)
    assert got.size == 48
    d = oracle.adamw_scalars(step, lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8,
                             weight_decay=0.1, grad_scale=grad_scale)
    want = np.array([d[k] for k in ("s", "b1", "c1", "b2", "c2", "bc1", "bc2", "lr", "eps", "d")],
                    np.float32)
    assert np.array_equal(got[:40].view(np.uint32), want.view(np.uint32))
    assert got[40:].view(np.float64)[0] == grad_scale
    with pytest.raises(ValueError):
        zs.zero_step_consts_make(zs.AdamWHParams(step=0))
    assert L.zero_step_consts_make(ctypes.byref(_hp()), None) == zs.ZERO_EINVAL


@cpu_only
def test_device_consts_entry_points_reject_bad_arguments():
    lay = zs.zero_flatten_layout([4096], 4)[0]
    S = L.zero_shard_step_dc
    args = [P(BASE), 0, 1024, 1024, P(BASE + (1 << 30)), P(BASE + (2 << 30)), P(BASE + (3 << 30)),
            P(BASE + (4 << 30)), 0, ctypes.byref(lay), 1, 0]
    tail = [None, None, None, 0, None]
    assert S(*args, None, *tail) == zs.ZERO_EINVAL                        # no constants
    assert S(*args, P(BASE + (5 << 30) + 4), *tail) == zs.ZERO_EINVAL     # not 8-byte aligned
    assert S(*args, P(BASE + (1 << 30) + 64), *tail) == zs.ZERO_EALIAS    # inside master
    assert S(*args, P(BASE + (4 << 30) + 2048 + 8), *tail) == zs.ZERO_EALIAS  # inside the slot
    assert S(P(0), 0, 1024, 0, *args[4:], P(0), *tail) == zs.ZERO_EINVAL  # NULL even when empty
    A = L.zero_shard_adamw_dc
    base = [P(BASE), P(BASE + (1 << 30)), P(BASE + (2 << 30)), P(BASE + (3 << 30)),
            P(BASE + (4 << 30)), 0, ctypes.byref(lay), 1, 0, 1024]
    assert A(*base, None, None, None) == zs.ZERO_EINVAL
    assert A(*base, P(BASE + (5 << 30) + 4), None, None) == zs.ZERO_EINVAL
    assert A(*base, P(BASE + (3 << 30) + 400), None, None) == zs.ZERO_EALIAS  # inside v
    lay8 = zs.zero_flatten_layout([8 * 4096], 8, 256)[0]
    C, V_ = L.zero_step_consts_select, L.zero_step_counter_advance
    tab, cnt, ctr = P(BASE + (8 << 30)), 10, P(BASE + (9 << 30))
    assert C(None, tab, cnt, ctr, None) == zs.ZERO_EINVAL
    assert C(P(BASE + (7 << 30)), None, cnt, ctr, None) == zs.ZERO_EINVAL
    assert C(P(BASE + (7 << 30)), tab, 0, ctr, None) == zs.ZERO_EINVAL          # empty table
    assert C(P(BASE + (7 << 30)), tab, cnt, None, None) == zs.ZERO_EINVAL
    assert C(P(BASE + (7 << 30) + 4), tab, cnt, ctr, None) == zs.ZERO_EINVAL    # unaligned
    assert C(P(BASE + (8 << 30) + 96), tab, cnt, ctr, None) == zs.ZERO_EALIAS   # inside the table
    assert C(P(BASE + (9 << 30) - 8), tab, cnt, ctr, None) == zs.ZERO_EALIAS    # over the counter
    assert C(P(BASE + (7 << 30)), tab, cnt, P(BASE + (9 << 30) + 4), None) == zs.ZERO_EINVAL
    assert V_(None, None, None) == zs.ZERO_EINVAL
    assert V_(P(BASE + (9 << 30) + 4), None, None) == zs.ZERO_EINVAL           # unaligned counter
    assert V_(ctr, P(BASE + (9 << 30) + 4), None) == zs.ZERO_EALIAS             # flag in counter
    Q = L.zero_shard_step_q8_dc
    q8 = [P(BASE), P(BASE + (1 << 28)), 4096, 16, 4096, P(BASE + (2 << 28)), P(BASE + (3 << 28)),
          P(BASE + (4 << 28)), P(BASE + (5 << 28)), P(BASE + (6 << 28)), ctypes.byref(lay8), 1, 0]
    qtail = [None, None, None, 0, None]
    assert Q(*q8, None, *qtail) == zs.ZERO_EINVAL
    assert Q(*q8, P(BASE + (7 << 28) + 4), *qtail) == zs.ZERO_EINVAL          # not 8-byte aligned
    assert Q(*q8, P(BASE + (4 << 28) + 64), *qtail) == zs.ZERO_EALIAS         # inside v
    assert Q(*q8, P(BASE + (6 << 28) + 16 * 4 + 8), *qtail) == zs.ZERO_EALIAS  # in the scale slot


def _pc(*pieces):
    arr = (zs._Piece * max(1, len(pieces)))()
    for i, (ptr, off, ln) in enumerate(pieces):
        arr[i] = zs._Piece(ptr, off, ln)
    return arr, len(pieces)


@cpu_only
def test_flat_copies_reject_bad_arguments():
    G, S, RS = L.zero_flat_gather, L.zero_flat_scatter, L.zero_reshard
    dst = P(BASE + (8 << 30))
    ok, n_ok = _pc((BASE, 0, 100), (BASE + 4096, 100, 50))
    assert G(ok, n_ok, 150, 3, 0, 10, dst, None) == zs.ZERO_EINVAL             # elem size 3
    assert G(ok, n_ok, -1, 4, 0, 10, dst, None) == zs.ZERO_EINVAL              # n < 0
    assert G(ok, n_ok, 150, 4, -1, 10, dst, None) == zs.ZERO_EINVAL            # begin < 0
    assert G(ok, n_ok, 150, 4, 0, -1, dst, None) == zs.ZERO_EINVAL             # count < 0
    assert G(ok, n_ok, 150, 4, 0, (1 << 38) + 1, dst, None) == zs.ZERO_EINVAL  # too long
    assert G(ok, n_ok, 150, 4, (1 << 63) - 5, 10, dst, None) == zs.ZERO_EINVAL  # index overflow
    assert G(ok, n_ok, 150, 4, 0, 10, None, None) == zs.ZERO_EINVAL
    assert G(ok, n_ok, 150, 4, 0, 10, P(BASE + (8 << 30) + 2), None) == zs.ZERO_EINVAL  # misaligned
    assert G(None, 2, 150, 4, 0, 10, dst, None) == zs.ZERO_EINVAL
    ov, n_ov = _pc((BASE, 0, 100), (BASE + 4096, 99, 50))                      # flat overlap
    assert G(ov, n_ov, 150, 4, 0, 10, dst, None) == zs.ZERO_EINVAL
    nul, n_nul = _pc((None, 0, 100),)
    assert G(nul, n_nul, 150, 4, 0, 10, dst, None) == zs.ZERO_EINVAL
    mis, n_mis = _pc((BASE + 2, 0, 100),)
    assert G(mis, n_mis, 150, 4, 0, 10, dst, None) == zs.ZERO_EINVAL
    neg, n_neg = _pc((BASE, -5, 100),)
    assert G(neg, n_neg, 150, 4, 0, 10, dst, None) == zs.ZERO_EINVAL
    assert G(ok, n_ok, 150, 4, 0, 10, P(BASE + 396), None) == zs.ZERO_EALIAS   # dst on a piece
    # empty requests need no buffers; empty pieces may be NULL
    assert G(ok, n_ok, 150, 4, 0, 0, None, None) == zs.ZERO_OK
    emp, n_emp = _pc((None, 0, 0), (None, 0, 0))
    assert G(emp, n_emp, 150, 4, 0, 0, None, None) == zs.ZERO_OK
    src = P(BASE + (9 << 30))
    assert S(src, 0, 10, ov, n_ov, 4, None) == zs.ZERO_EINVAL
    mem, n_mem = _pc((BASE, 0, 100), (BASE + 200, 100, 50))                    # memory overlap
    assert S(src, 0, 10, mem, n_mem, 4, None) == zs.ZERO_EALIAS
    assert S(P(BASE + 40), 0, 10, ok, n_ok, 4, None) == zs.ZERO_EALIAS          # src in a piece
    assert S(None, 0, 10, ok, n_ok, 4, None) == zs.ZERO_EINVAL
    assert S(None, 0, 0, ok, n_ok, 4, None) == zs.ZERO_OK
    sh = (P * 2)(P(BASE), P(BASE + (1 << 30)))
    assert RS(sh, 0, 100, 150, 4, 0, 75, dst, None) == zs.ZERO_EINVAL          # no old shards
    assert RS(sh, 2, 100, 201, 4, 0, 75, dst, None) == zs.ZERO_EINVAL          # n > n_src * shard
    assert RS(sh, 2, -1, 0, 4, 0, 75, dst, None) == zs.ZERO_EINVAL
    assert RS(sh, 2, 100, 150, 4, -1, 75, dst, None) == zs.ZERO_EINVAL
    assert RS(sh, 2, 100, 150, 4, 1, -75, dst, None) == zs.ZERO_EINVAL
    assert RS(sh, 2, 100, 150, 4, 0, 75, P(BASE + 40), None) == zs.ZERO_EALIAS
    assert RS(sh, 2, 100, 150, 4, 0, 0, None, None) == zs.ZERO_OK


@pytest.mark.parametrize("seed", range(25))
def test_dim0_layout_and_segments_match_oracle(seed):
    rng = np.random.default_rng(500 + seed)
    shapes = [(int(rng.integers(0, 70)), int(rng.choice([0, 1, 3, 16, 4096])))
              for _ in range(int(rng.integers(0, 14)))]
    n_dp = int(rng.integers(1, 70))
    align = int(rng.choice([1, 4, 8]))
    lay, offs, chunk = zs.zero_dim0_layout(shapes, n_dp, align)
    o_offs, o_chunk, n, s = oracle.dim0_layout(shapes, n_dp, align)
    assert (lay.n, lay.shard, lay.n_pad, lay.n_dp, lay.align) == (n, s, n_dp * s, n_dp, align)
    assert np.array_equal(offs, o_offs) and np.array_equal(chunk, o_chunk)
    for rank in sorted({0, n_dp - 1, int(rng.integers(0, n_dp))}):
        want = [q for q in oracle.dim0_segments(shapes, n_dp, rank, align) if q[3] > 0]
        assert zs.zero_dim0_segments(lay, shapes, rank) == want


def test_dim0_llama7b_is_the_flat_shard_size():
    d, ffn, vocab = 4096, 11008, 32000
    shapes = [(vocab, d)] + [(d, d)] * 4 * 32 + [(ffn, d)] * 64 + [(d, ffn)] * 32 + \
        [(d, 1)] * 65 + [(vocab, d)]
    lay, _, _ = zs.zero_dim0_layout(shapes, 8)
    flat, _ = zs.zero_flatten_layout(llama7b_numels(), 8)
    assert (lay.n, lay.shard, lay.n_pad) == (flat.n, flat.shard, flat.n_pad)


def test_dim0_rejects_invalid():
    with pytest.raises(zs.ZeroError):
        zs.zero_dim0_layout([(4, -1)], 2)
    with pytest.raises(zs.ZeroError):
        zs.zero_dim0_layout([(4, 1)], 0)
    with pytest.raises(zs.ZeroError):
        zs.zero_dim0_layout([(4, 1)], 2, 0)
    with pytest.raises(zs.ZeroError):
        zs.zero_dim0_layout([(1 << 62, 4)], 2)  # numel overflows
    lay, _, _ = zs.zero_dim0_layout([(10, 3)], 4)
    with pytest.raises(zs.ZeroError):
        zs.zero_dim0_segments(lay, [(10, 4)], 0)  # inconsistent with the layout
    with pytest.raises(zs.ZeroError):
        zs.zero_dim0_segments(lay, [(10, 3)], 4)  # rank out of range


@cpu_only
def test_fp32_rows_validation():
    R = L.zero_shard_reduce
    # fp32 rows: 4 bytes per element in the alias check (16-bit would miss it)
    assert R(P(BASE), 2, 2, 16, 16, P(BASE + 100), 0, None, None, None, 0,
             None) == zs.ZERO_EALIAS
    assert R(P(BASE), 3, 2, 16, 16, P(BASE + 4096), 0, None, None, None, 0,
             None) == zs.ZERO_EINVAL
    # weights cannot be fp32
    assert _step(wdt=2) == zs.ZERO_EINVAL
    assert _step(gdt=2, v=BASE + 3 * 1024 * 4 - 8) == zs.ZERO_EALIAS  # v over the fp32 rows


@cpu_only
def test_q8_entry_points_reject_bad_arguments():
    Q, D, S8 = L.zero_q8_quantize, L.zero_q8_dequantize, L.zero_shard_step_q8
    assert Q(P(BASE), 3, 100, P(BASE + 4096), P(BASE + 8192), None) == zs.ZERO_EINVAL
    assert Q(P(BASE), 2, -1, P(BASE + 4096), P(BASE + 8192), None) == zs.ZERO_EINVAL
    assert Q(None, 2, 100, P(BASE + 4096), P(BASE + 8192), None) == zs.ZERO_EINVAL
    assert Q(P(BASE), 2, 1000, P(BASE + 100), P(BASE + 8192), None) == zs.ZERO_EALIAS
    assert Q(P(BASE), 2, 1000, P(BASE + 8192), P(BASE + 8192 + 500), None) == zs.ZERO_EALIAS
    assert Q(None, 2, 0, None, None, None) == zs.ZERO_OK
    assert D(P(BASE), P(BASE + 4096), 1000, P(BASE + 500), 0, None) == zs.ZERO_EALIAS
    assert D(P(BASE), P(BASE + 4096), 1000, P(BASE + 8192), 7, None) == zs.ZERO_EINVAL
    lay = zs.zero_flatten_layout([8 * 4096], 8, 256)[0]
    hp = _hp()

    def step(gq=BASE, gs=BASE + (1 << 28), ld=4096, sld=16, length=4096, w=BASE + (2 << 28),
             m=BASE + (3 << 28), v=BASE + (4 << 28), wq=BASE + (5 << 28), ws=BASE + (6 << 28),
             lay=lay, rank=1, off=0, ssq=None, wk=None, wk_bytes=0):
        return S8(P(gq), P(gs), ld, sld, length, P(w), P(m), P(v), P(wq), P(ws),
                  ctypes.byref(lay), rank, off, ctypes.byref(hp), None,
                  P(ssq) if ssq else None, P(wk) if wk else None, wk_bytes, None)
    assert step(off=128) == zs.ZERO_EINVAL                          # not a block boundary
    assert step(sld=15) == zs.ZERO_EINVAL                           # scale rows too short
    assert step(ld=4098) == zs.ZERO_EINVAL                          # row stride not % 4
    assert step(gq=BASE + 2) == zs.ZERO_EINVAL                      # codes misaligned
    assert step(ld=1 << 60) == zs.ZERO_EINVAL                       # code rows past 2^60
    assert step(sld=1 << 59) == zs.ZERO_EINVAL                      # scale rows past 2^60
    assert step(w=BASE + (2 << 28) + 4) == zs.ZERO_EINVAL           # master misaligned
    assert step(length=4096, off=256) == zs.ZERO_ERANGE
    odd = zs.zero_flatten_layout([8 * 4000], 8)[0]                  # shard 4000: not % 256
    assert step(lay=odd, length=1000) == zs.ZERO_EINVAL
    assert step(m=BASE + (2 << 28) + 16 * 1000) == zs.ZERO_EALIAS   # m inside master
    assert step(ws=BASE + (1 << 28) + 64) == zs.ZERO_EALIAS         # scale slot over row scales
    assert step(w=BASE + 7 * 4096) == zs.ZERO_EALIAS                # master over the last row
    assert step(length=0, gq=0, gs=0, w=0, m=0, v=0, wq=0, ws=0) == zs.ZERO_OK
    wkb = zs.zero_sumsq_workspace_bytes(4096)
    assert step(ssq=BASE + (7 << 28)) == zs.ZERO_EINVAL             # sum without workspace
    assert step(ssq=BASE + (7 << 28), wk=BASE + (7 << 28) + 4096,
                wk_bytes=wkb - 1) == zs.ZERO_EINVAL                  # workspace too small
    assert step(ssq=BASE + (7 << 28), wk=BASE + (4 << 28),
                wk_bytes=wkb) == zs.ZERO_EALIAS                      # workspace over v


@cpu_only
def test_noalloc_step_rejects_before_any_launch():
    """zero_shard_step_noalloc: with a sum of squares, a range longer than
    the library's scratch covers is refused; other arguments are checked as
    zero_shard_step checks them."""
    lay = zs.zero_flatten_layout([4096], 4)[0]
    big = (1 << 29) + 4

    def call(length=1024, ld=1024, rank=1, ssq=None):
        return L.zero_shard_step_noalloc(P(BASE), 0, ld, length, P(BASE + (1 << 30)),
                                         P(BASE + (2 << 30)), P(BASE + (3 << 30)),
                                         P(BASE + (4 << 30)), 0, ctypes.byref(lay), rank, 0,
                                         ctypes.byref(_hp()), None, P(ssq) if ssq else None,
                                         None)
    assert zs.ZERO_NOALLOC_MAX_LEN == 1 << 29
    assert call(length=big, ld=big, ssq=BASE + (6 << 30)) == zs.ZERO_EINVAL
    assert call(rank=4) == zs.ZERO_EINVAL
    assert call(ld=1000) == zs.ZERO_EINVAL
    assert call(length=1025, ld=1025) == zs.ZERO_ERANGE


@pytest.mark.parametrize("seed", range(4))
def test_array_split_layout_matches_numpy_and_the_oracle(seed):
    """zero_array_split_layout cuts as numpy.array_split (a library routine)
    cuts; the oracle's piece starts agree, also far beyond 2^32 elements."""
    rng = np.random.default_rng(seed)
    cases = [(0, 1), (0, 5), (3, 8), (7, 7), (10_000, 4), (10_001, 4)]
    cases += [(int(rng.integers(0, 50_000)), int(rng.integers(1, 130))) for _ in range(60)]
    for n, n_dp in cases:
        starts, lens = zs.zero_array_split_layout(n, n_dp)
        pieces = np.array_split(np.arange(n), n_dp)
        assert lens.tolist() == [p.size for p in pieces]
        assert starts.tolist() == [int(p[0]) if p.size else int(s) for p, s in zip(pieces, starts)]
        assert np.array_equal(np.concatenate([np.arange(s, s + l) for s, l in zip(starts, lens)]
                                             + [np.zeros(0, np.int64)]), np.arange(n))
    for n, n_dp in [(6_738_415_616, 8), ((1 << 40) + 12_345, 64), (1_557_611_200, 3)]:
        starts, lens = zs.zero_array_split_layout(n, n_dp)
        assert starts.tolist() == [oracle.array_split_start(n, n_dp, r) for r in range(n_dp)]
        assert int(lens.sum()) == n and starts[-1] + lens[-1] == n


def test_array_split_layout_rejects_invalid():
    for n, n_dp in [(-1, 4), (10, 0), (10, -3)]:
        with pytest.raises(zs.ZeroValueError):
            zs.zero_array_split_layout(n, n_dp)
    assert L.zero_array_split_layout(10, 4, None, None) == zs.ZERO_EINVAL
