"""Seeded synthetic inputs, shared by the tests, the benchmark and the smoke
check.  Holds no arithmetic of the optimizer step: it only draws values
(see synth_core.h for the definition) on the host or straight into device
memory.  The workload definitions live in synth.workloads.
"""
import ctypes
import os

import numpy as np

from .synth_const import F32, BF16, F16, TABLE_SIZE, outlier_threshold, tag  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
# SYNTH_LIB selects another build of synth_cpu.c (the sanitizer tests load
# an AddressSanitizer/UBSan build this way)
LIB_CPU = os.environ.get("SYNTH_LIB") or os.path.join(HERE, "libsynth.so")
LIB_GPU = os.path.join(HERE, "libsynth_gpu.so")

_cpu = None
_gpu = None
_table = None
_dev_tables = {}


def host_threads():
    """Threads for host generation: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _cpu_lib():
    global _cpu
    if _cpu is None:
        if not os.path.exists(LIB_CPU):
            raise ImportError(f"{LIB_CPU} is not built: run synth/build.py")
        L = ctypes.CDLL(LIB_CPU)
        vp = ctypes.c_void_p
        L.syn_table.argtypes = [vp]
        L.syn_table.restype = None
        common = [ctypes.c_double, ctypes.c_uint32, ctypes.c_double, vp, vp, ctypes.c_int]
        L.syn_fill.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                               ctypes.c_int64, ctypes.c_int64] + common
        L.syn_fill.restype = ctypes.c_int
        L.syn_gather.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64, vp,
                                 ctypes.c_int64] + common
        L.syn_gather.restype = ctypes.c_int
        _cpu = L
    return _cpu


def table():
    """The quantile table (float64[TABLE_SIZE]); both builds index this array."""
    global _table
    if _table is None:
        t = np.zeros(TABLE_SIZE, dtype=np.float64)
        _cpu_lib().syn_table(t.ctypes.data_as(ctypes.c_void_p))
        _table = t
    return _table


def _np_dtype(kind):
    return np.float32 if kind == F32 else np.uint16


def fill_host(kind, seed, tg, start, count, sigma, thr=0, mul=1.0, out=None, nthreads=None):
    """Elements [start, start + count) of stream (seed, tg) on the host."""
    if out is None:
        out = np.empty(count, dtype=_np_dtype(kind))
    assert out.dtype == _np_dtype(kind) and out.flags.c_contiguous and out.size >= count
    t = table()
    rc = _cpu_lib().syn_fill(kind, seed, tg, start, count, sigma, thr, mul,
                             t.ctypes.data_as(ctypes.c_void_p),
                             out.ctypes.data_as(ctypes.c_void_p),
                             nthreads or host_threads())
    if rc != 0:
        raise RuntimeError("syn_fill failed")
    return out


def gather_host(kind, seed, tg, idx, sigma, thr=0, mul=1.0, nthreads=None):
    """Elements idx[...] of stream (seed, tg) on the host."""
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=_np_dtype(kind))
    t = table()
    rc = _cpu_lib().syn_gather(kind, seed, tg, idx.ctypes.data_as(ctypes.c_void_p),
                               idx.size, sigma, thr, mul,
                               t.ctypes.data_as(ctypes.c_void_p),
                               out.ctypes.data_as(ctypes.c_void_p),
                               nthreads or host_threads())
    if rc != 0:
        raise RuntimeError("syn_gather failed")
    return out


def _gpu_lib():
    global _gpu
    if _gpu is None:
        if not os.path.exists(LIB_GPU):
            raise ImportError(f"{LIB_GPU} is not built: run synth/build.py")
        import torch  # noqa: F401  (its HIP runtime first: one runtime per process)
        L = ctypes.CDLL(LIB_GPU)
        vp = ctypes.c_void_p
        L.syn_gpu_fill.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                   ctypes.c_uint32, ctypes.c_double, vp, vp, vp]
        L.syn_gpu_fill.restype = ctypes.c_int
        _gpu = L
    return _gpu


def fill_device(dst, kind, seed, tg, start, sigma, thr=0, mul=1.0, stream=None):
    """Fill the contiguous torch tensor dst (on a GPU) with elements
    [start, start + dst.numel()) of stream (seed, tg)."""
    import torch
    want = torch.float32 if kind == F32 else (torch.bfloat16 if kind == BF16 else torch.float16)
    if dst.dtype not in (want, torch.int16, torch.uint16) or not dst.is_contiguous() or not dst.is_cuda:
        raise TypeError("fill_device: dst must be a contiguous CUDA tensor of the drawn type")
    if kind == F32 and dst.dtype != torch.float32:
        raise TypeError("fill_device: float32 draws need a float32 tensor")
    dev = dst.device.index if dst.device.index is not None else torch.cuda.current_device()
    if dev not in _dev_tables:
        _dev_tables[dev] = torch.from_numpy(table()).to(dst.device)
    tab = _dev_tables[dev]
    if stream is None:
        stream = torch.cuda.current_stream(dst.device).cuda_stream
    rc = _gpu_lib().syn_gpu_fill(kind, seed, tg, start, dst.numel(), sigma, thr, mul,
                                 ctypes.c_void_p(tab.data_ptr()),
                                 ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"syn_gpu_fill failed ({rc})")
    return dst
