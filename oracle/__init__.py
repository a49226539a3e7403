"""ctypes wrapper for the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import this package.  It works on numpy arrays on the host and never touches
a GPU.  Arrays holding 16-bit values are numpy uint16 (raw bit patterns).
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB selects another build of oracle_zero.c (the mutation tests load
# deliberately broken copies to show that the pins catch them)
LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(HERE, "liboracle_zero.so")

BF16, FP16, FP32 = 0, 1, 2

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run oracle/build.py")
        L = ctypes.CDLL(LIB_PATH)
        i64p = ctypes.POINTER(ctypes.c_int64)
        vp = ctypes.c_void_p
        L.ora_flatten_layout.argtypes = [i64p, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int64, i64p, i64p]
        L.ora_flatten_layout.restype = ctypes.c_int
        L.ora_shard_segments.argtypes = [i64p, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.c_int32, i64p,
                                         ctypes.c_int64]
        L.ora_shard_segments.restype = ctypes.c_int64
        L.ora_array_split_start.argtypes = [ctypes.c_int64] * 3
        L.ora_array_split_start.restype = ctypes.c_int64
        for name in ("ora_f32_to_bf16_n", "ora_f32_to_f16_n",
                     "ora_bf16_to_f32_n", "ora_f16_to_f32_n"):
            getattr(L, name).argtypes = [vp, vp, ctypes.c_int64]
            getattr(L, name).restype = None
        L.ora_adamw_scalars.argtypes = [vp, ctypes.c_int64, vp]
        L.ora_adamw_scalars.restype = None
        L.ora_reduce.argtypes = [vp, ctypes.c_int, ctypes.c_int32, ctypes.c_int64,
                                 ctypes.c_int64, vp, ctypes.c_int, vp, vp]
        L.ora_reduce.restype = None
        L.ora_adamw.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int64,
                                vp, ctypes.c_int64, vp]
        L.ora_adamw.restype = None
        L.ora_step.argtypes = [vp, ctypes.c_int, ctypes.c_int32, ctypes.c_int64,
                               ctypes.c_int64, vp, vp, vp, vp, ctypes.c_int, vp,
                               ctypes.c_int64, vp, vp]
        L.ora_step.restype = None
        L.ora_clip_coef.argtypes = [ctypes.c_double, ctypes.c_float, ctypes.c_double]
        L.ora_clip_coef.restype = ctypes.c_float
        L.ora_adamw_ex.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int64, vp,
                                   ctypes.c_int64, vp, vp, ctypes.c_double, vp]
        L.ora_adamw_ex.restype = None
        L.ora_loss_scale_update.argtypes = [vp, vp, ctypes.c_uint32, ctypes.c_double,
                                            ctypes.c_double, ctypes.c_int32]
        L.ora_loss_scale_update.restype = None
        L.ora_reshard.argtypes = [vp, ctypes.c_int32, ctypes.c_int64, vp, ctypes.c_int64,
                                  ctypes.c_int32, ctypes.c_int64, ctypes.c_int32]
        L.ora_reshard.restype = None
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.ora_dim0_layout.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                      vp, vp, vp]
        L.ora_dim0_layout.restype = ctypes.c_int
        L.ora_dim0_segments.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                        ctypes.c_int32, vp, ctypes.c_int64]
        L.ora_dim0_segments.restype = ctypes.c_int64
        L.ora_flat_locate.argtypes = [i64p, i64p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                      i64p]
        L.ora_flat_locate.restype = ctypes.c_int32
        L.ora_flat_gather.argtypes = [vp, i64p, i64p, ctypes.c_int32, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int64, vp, ctypes.c_int32]
        L.ora_flat_gather.restype = None
        L.ora_flat_scatter.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, vp, i64p, i64p,
                                       ctypes.c_int32, ctypes.c_int32]
        L.ora_flat_scatter.restype = None
        L.ora_q8_quantize.argtypes = [vp, ctypes.c_int, ctypes.c_int64, vp, vp]
        L.ora_q8_quantize.restype = None
        L.ora_q8_dequantize.argtypes = [vp, vp, ctypes.c_int64, vp, ctypes.c_int]
        L.ora_q8_dequantize.restype = None
        L.ora_step_q8.argtypes = [vp, vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int64, vp, vp, vp, vp, vp, vp, ctypes.c_int64, vp, vp]
        L.ora_step_q8.restype = None
        L.ora_model_state_bytes.argtypes = [ctypes.c_double, ctypes.c_double,
                                            ctypes.c_int, ctypes.c_double]
        L.ora_model_state_bytes.restype = ctypes.c_double
        L.ora_comm_bytes.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_int,
                                     ctypes.c_double, ctypes.c_double]
        L.ora_comm_bytes.restype = ctypes.c_double
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _need(a, dtype, name):
    if not (isinstance(a, np.ndarray) and a.dtype == dtype and a.flags.c_contiguous):
        raise TypeError(f"{name}: need a C-contiguous numpy {np.dtype(dtype).name} array")


def flatten_layout(numels, n_dp, align=1):
    """-> (offsets, N, N_pad, S) or raises ValueError."""
    nums = np.ascontiguousarray(numels, dtype=np.int64)
    offs = np.zeros(len(nums), dtype=np.int64)
    out = np.zeros(3, dtype=np.int64)
    rc = lib().ora_flatten_layout(
        nums.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(nums), n_dp, align,
        offs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    if rc != 0:
        raise ValueError("invalid layout arguments")
    return offs, int(out[0]), int(out[1]), int(out[2])


def shard_segments(numels, n_dp, rank, align=1):
    """-> list of (tensor, tensor_off, shard_off, len); tensor -1 is padding."""
    nums = np.ascontiguousarray(numels, dtype=np.int64)
    p = nums.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    cnt = lib().ora_shard_segments(p, len(nums), n_dp, align, rank, None, 0)
    if cnt < 0:
        raise ValueError("invalid segment arguments")
    q = np.zeros(4 * max(cnt, 1), dtype=np.int64)
    lib().ora_shard_segments(p, len(nums), n_dp, align, rank,
                             q.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), cnt)
    return [tuple(int(x) for x in q[4 * i:4 * i + 4]) for i in range(cnt)]


def dim0_layout(shapes, n_dp, align=1):
    """shapes: [(rows, cols), ...] -> (packed_off, chunk_rows, N, S)."""
    rows = np.ascontiguousarray([r for r, _ in shapes], dtype=np.int64)
    cols = np.ascontiguousarray([c for _, c in shapes], dtype=np.int64)
    offs = np.zeros(max(1, len(shapes)), dtype=np.int64)
    chunk = np.zeros(max(1, len(shapes)), dtype=np.int64)
    out = np.zeros(2, dtype=np.int64)
    if lib().ora_dim0_layout(_ptr(rows), _ptr(cols), len(shapes), n_dp, align, _ptr(offs),
                             _ptr(chunk), _ptr(out)) != 0:
        raise ValueError("invalid dim-0 layout arguments")
    return offs[:len(shapes)], chunk[:len(shapes)], int(out[0]), int(out[1])


def dim0_segments(shapes, n_dp, rank, align=1):
    """(tensor, tensor_off, shard_off, len) pieces of rank's packed buffer."""
    rows = np.ascontiguousarray([r for r, _ in shapes], dtype=np.int64)
    cols = np.ascontiguousarray([c for _, c in shapes], dtype=np.int64)
    cnt = lib().ora_dim0_segments(_ptr(rows), _ptr(cols), len(shapes), n_dp, align, rank,
                                  None, 0)
    if cnt < 0:
        raise ValueError("invalid dim-0 segment arguments")
    q = np.zeros(4 * max(cnt, 1), dtype=np.int64)
    lib().ora_dim0_segments(_ptr(rows), _ptr(cols), len(shapes), n_dp, align, rank, _ptr(q),
                            cnt)
    return [tuple(int(x) for x in q[4 * i:4 * i + 4]) for i in range(cnt)]


def array_split_start(n, parts, i):
    return lib().ora_array_split_start(n, parts, i)


def f32_to_bf16(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    lib().ora_f32_to_bf16_n(_ptr(x), _ptr(y), x.size)
    return y


def f32_to_f16(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    lib().ora_f32_to_f16_n(_ptr(x), _ptr(y), x.size)
    return y


def bf16_to_f32(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    y = np.empty(h.shape, dtype=np.float32)
    lib().ora_bf16_to_f32_n(_ptr(h), _ptr(y), h.size)
    return y


def f16_to_f32(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    y = np.empty(h.shape, dtype=np.float32)
    lib().ora_f16_to_f32_n(_ptr(h), _ptr(y), h.size)
    return y


def _hp(lr, beta1, beta2, eps, weight_decay, grad_scale):
    return np.array([lr, beta1, beta2, eps, weight_decay, grad_scale], dtype=np.float64)


def adamw_scalars(step, lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1,
                  grad_scale=1.0):
    """-> dict of the fp32 scalars s, b1, c1, b2, c2, bc1, bc2, lr, eps, d."""
    hp = _hp(lr, beta1, beta2, eps, weight_decay, grad_scale)
    out = np.zeros(10, dtype=np.float32)
    lib().ora_adamw_scalars(_ptr(hp), step, _ptr(out))
    keys = ("s", "b1", "c1", "b2", "c2", "bc1", "bc2", "lr", "eps", "d")
    return dict(zip(keys, (np.float32(v) for v in out)))


def reduce(grads, gdt, n_contrib, ld, length, acc, accumulate, overflow=None, sumsq=None):
    """In place on acc (float32[length]); overflow uint32[1]; sumsq float64[1].
    grads: uint16 rows (BF16, FP16) or float32 rows (FP32)."""
    _need(grads, np.float32 if gdt == FP32 else np.uint16, "grads")
    _need(acc, np.float32, "acc")
    if length > 0 and grads.size < (n_contrib - 1) * ld + length:
        raise ValueError("grads too small")
    lib().ora_reduce(_ptr(grads), gdt, n_contrib, ld, length, _ptr(acc),
                     int(bool(accumulate)), _ptr(overflow), _ptr(sumsq))


def adamw(acc, w, m, v, wout, wdt, length, step, lr=1e-4, beta1=0.9, beta2=0.999,
          eps=1e-8, weight_decay=0.1, grad_scale=1.0, skip=None):
    """In place on w, m, v (float32) and wout (uint16)."""
    for a, n in ((acc, "acc"), (w, "w"), (m, "m"), (v, "v")):
        _need(a, np.float32, n)
    _need(wout, np.uint16, "wout")
    hp = _hp(lr, beta1, beta2, eps, weight_decay, grad_scale)
    lib().ora_adamw(_ptr(acc), _ptr(w), _ptr(m), _ptr(v), _ptr(wout), wdt, length,
                    _ptr(hp), step, _ptr(skip))


def clip_coef(sumsq, s, max_norm):
    return float(np.float32(lib().ora_clip_coef(float(sumsq), float(s), float(max_norm))))


def adamw_ex(acc, w, m, v, wout, wdt, length, step, lr=1e-4, beta1=0.9, beta2=0.999,
             eps=1e-8, weight_decay=0.1, grad_scale=1.0, skip=None, sumsq=None, max_norm=0.0,
             loss_scale=None):
    """adamw with clipping (sumsq float64[1], max_norm) and a dynamic loss scale
    (loss_scale float32[1]: s = grad_scale / loss_scale)."""
    for a, n in ((acc, "acc"), (w, "w"), (m, "m"), (v, "v")):
        _need(a, np.float32, n)
    _need(wout, np.uint16, "wout")
    hp = _hp(lr, beta1, beta2, eps, weight_decay, grad_scale)
    lib().ora_adamw_ex(_ptr(acc), _ptr(w), _ptr(m), _ptr(v), _ptr(wout), wdt, length, _ptr(hp),
                       step, _ptr(skip), _ptr(sumsq), float(max_norm), _ptr(loss_scale))


def loss_scale_update(scale, good_steps, overflow, growth=2.0, backoff=0.5, interval=2000):
    """In place on scale (float32[1]) and good_steps (int32[1])."""
    _need(scale, np.float32, "scale")
    _need(good_steps, np.int32, "good_steps")
    lib().ora_loss_scale_update(_ptr(scale), _ptr(good_steps), int(overflow), float(growth),
                                float(backoff), int(interval))


def step(grads, gdt, n_dp, ld, length, w, m, v, wout, wdt, step, lr=1e-4, beta1=0.9,
         beta2=0.999, eps=1e-8, weight_decay=0.1, grad_scale=None, overflow=None,
         sumsq=None):
    """Fused reduce + AdamW + cast, in place on w, m, v, wout.

    grad_scale defaults to 1/n_dp, the average over ranks."""
    _need(grads, np.float32 if gdt == FP32 else np.uint16, "grads")
    for a, n in ((w, "w"), (m, "m"), (v, "v")):
        _need(a, np.float32, n)
    _need(wout, np.uint16, "wout")
    if length > 0 and grads.size < (n_dp - 1) * ld + length:
        raise ValueError("grads too small")
    if grad_scale is None:
        grad_scale = 1.0 / n_dp
    hp = _hp(lr, beta1, beta2, eps, weight_decay, grad_scale)
    lib().ora_step(_ptr(grads), gdt, n_dp, ld, length, _ptr(w), _ptr(m), _ptr(v),
                   _ptr(wout), wdt, _ptr(hp), step, _ptr(overflow), _ptr(sumsq))


def reshard(src_shards, n, dst_n_dp, dst_rank, dst_align=1):
    """New rank dst_rank's shard (for dst_n_dp ranks) of the flat vector held
    as the list of old shards src_shards (equal length numpy arrays)."""
    src = [np.ascontiguousarray(a) for a in src_shards]
    dt = src[0].dtype
    assert all(a.dtype == dt and a.size == src[0].size for a in src)
    _, _, _, dst_shard = flatten_layout([n], dst_n_dp, dst_align)
    dst = np.empty(dst_shard, dtype=dt)
    ptrs = (ctypes.c_void_p * len(src))(*[a.ctypes.data for a in src])
    lib().ora_reshard(ptrs, len(src), src[0].size, _ptr(dst), dst_shard, dst_rank, n,
                      dt.itemsize)
    return dst


def _i64s(xs):
    return (ctypes.c_int64 * max(1, len(xs)))(*[int(x) for x in xs])


def flat_locate(pieces, n, i):
    """(k, off) of flat index i among pieces [(flat_off, len), ...], or
    (-1, None) when i >= n or no piece holds it."""
    off = ctypes.c_int64(0)
    k = lib().ora_flat_locate(_i64s([p[0] for p in pieces]), _i64s([p[1] for p in pieces]),
                              len(pieces), n, i, ctypes.byref(off))
    return (k, off.value) if k >= 0 else (-1, None)


def flat_gather(sources, n, begin, count):
    """dst[j] = flat[begin + j], 0 outside the pieces or beyond n.
    sources: [(array, flat_off), ...], each array one piece."""
    arrs = [np.ascontiguousarray(a) for a, _ in sources]
    dt = arrs[0].dtype
    assert all(a.dtype == dt for a in arrs)
    dst = np.empty(count, dtype=dt)
    ptrs = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    lib().ora_flat_gather(ptrs, _i64s([o for _, o in sources]), _i64s([a.size for a in arrs]),
                          len(arrs), n, begin, count, _ptr(dst), dt.itemsize)
    return dst


def flat_scatter(src, begin, dests):
    """Writes src (flat indices [begin, begin + src.size)) into the pieces
    dests [(array, flat_off), ...] in place, where they hold those indices."""
    src = np.ascontiguousarray(src)
    for a, _ in dests:
        assert a.dtype == src.dtype and a.flags.c_contiguous
    ptrs = (ctypes.c_void_p * len(dests))(*[a.ctypes.data for a, _ in dests])
    lib().ora_flat_scatter(_ptr(src), begin, src.size, ptrs, _i64s([o for _, o in dests]),
                           _i64s([a.size for a, _ in dests]), len(dests), src.dtype.itemsize)


Q8_BLOCK = 256


def q8_blocks(length):
    return (length + Q8_BLOCK - 1) // Q8_BLOCK


def q8_quantize(x, xdt):
    """(int8 codes, float32 scales) of x (float32 with FP32, uint16 with BF16/FP16)."""
    _need(x, np.float32 if xdt == FP32 else np.uint16, "x")
    q = np.zeros(x.size, np.int8)
    s = np.zeros(max(1, q8_blocks(x.size)), np.float32)
    lib().ora_q8_quantize(_ptr(x), xdt, x.size, _ptr(q), _ptr(s))
    return q, s[:q8_blocks(x.size)]


def q8_dequantize(q, scales, ydt=FP32):
    _need(q, np.int8, "q")
    _need(scales, np.float32, "scales")
    y = np.zeros(q.size, np.float32 if ydt == FP32 else np.uint16)
    lib().ora_q8_dequantize(_ptr(q), _ptr(scales), q.size, _ptr(y), ydt)
    return y


def step_q8(gq, gs, n_dp, ld, sld, length, w, m, v, wq, wscales, step, lr=1e-4, beta1=0.9,
            beta2=0.999, eps=1e-8, weight_decay=0.1, grad_scale=None, overflow=None, sumsq=None):
    """Fused step with int8 rows (codes gq, scales gs) and int8 weights out."""
    _need(gq, np.int8, "gq")
    _need(gs, np.float32, "gs")
    _need(wq, np.int8, "wq")
    _need(wscales, np.float32, "wscales")
    for a, n in ((w, "w"), (m, "m"), (v, "v")):
        _need(a, np.float32, n)
    if grad_scale is None:
        grad_scale = 1.0 / n_dp
    hp = _hp(lr, beta1, beta2, eps, weight_decay, grad_scale)
    lib().ora_step_q8(_ptr(gq), _ptr(gs), n_dp, ld, sld, length, _ptr(w), _ptr(m), _ptr(v),
                      _ptr(wq), _ptr(wscales), _ptr(hp), step, _ptr(overflow), _ptr(sumsq))


def model_state_bytes(n, n_dp, stage, k=12):
    return lib().ora_model_state_bytes(float(n), float(n_dp), stage, float(k))


def comm_bytes(n, n_dp, stage, param_bytes=2, grad_bytes=2):
    return lib().ora_comm_bytes(float(n), float(n_dp), stage, float(param_bytes),
                                float(grad_bytes))
