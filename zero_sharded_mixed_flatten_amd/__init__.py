"""zero_sharded_mixed_flatten_amd -- one data-parallel rank's sharded,
mixed-precision optimizer step on MI355X (gfx950).

A thin ctypes binding over libzero_shard.so (include/zero_shard.h).  Every
function here has the name of the C entry point it calls and only marshals
arguments: torch tensors become device pointers and dtype codes, the current
torch stream becomes the HIP stream.  All work runs in the library's HIP
kernels; there is no fallback of any kind -- importing this package without
the built library raises ImportError.

    layout, offsets = zero_flatten_layout(numels, n_dp)
    hp = AdamWHParams(lr=1e-4, step=1, grad_scale=1 / n_dp)
    zero_shard_step(grads, ld, S, master, m, v, weight_full, layout, rank, hp)
"""
import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libzero_shard.so")

ZERO_OK, ZERO_EINVAL, ZERO_EALIAS, ZERO_ERANGE, ZERO_EDEVICE = range(5)
ZERO_BF16, ZERO_FP16, ZERO_FP32 = 0, 1, 2
ZERO_Q8_BLOCK = 256
ABI_VERSION = 4


class ZeroError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_lib.zero_status_string(status).decode()}")


class ZeroValueError(ZeroError, ValueError):
    """Invalid arguments (EINVAL, EALIAS, ERANGE): a ValueError, the pages'
    convention for an unsupported stage or argument."""


class ZeroLayout(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("n_pad", ctypes.c_int64), ("shard", ctypes.c_int64),
                ("align", ctypes.c_int64), ("n_dp", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]

    def __repr__(self):
        return (f"ZeroLayout(n={self.n}, n_pad={self.n_pad}, shard={self.shard}, "
                f"align={self.align}, n_dp={self.n_dp})")


class _HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("grad_scale", ctypes.c_double),
                ("step", ctypes.c_int64)]


class _StepControl(ctypes.Structure):
    _fields_ = [("skip", ctypes.c_void_p), ("sumsq", ctypes.c_void_p),
                ("max_norm", ctypes.c_double), ("loss_scale", ctypes.c_void_p)]


class ZeroStepConsts(ctypes.Structure):
    """zero_step_consts: the update's ten fp32 constants and grad_scale."""
    _fields_ = [(name, ctypes.c_float) for name in
                ("s", "b1", "c1", "b2", "c2", "bc1", "bc2", "lr", "eps", "d")] + \
               [("grad_scale", ctypes.c_double)]


class _Piece(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("flat_off", ctypes.c_int64), ("len", ctypes.c_int64)]


class _Segment(ctypes.Structure):
    _fields_ = [("tensor", ctypes.c_int64), ("tensor_off", ctypes.c_int64),
                ("shard_off", ctypes.c_int64), ("len", ctypes.c_int64)]


@dataclass
class AdamWHParams:
    """AdamW hyperparameters as the C struct takes them (doubles)."""
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.1
    grad_scale: float = 1.0
    step: int = 1

    def _c(self) -> _HParams:
        return _HParams(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay,
                        self.grad_scale, int(self.step))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950) first")
    # torch ships its own HIP runtime.  Loaded first, it is the one this
    # library binds to (same soname); loaded after this library it would be
    # a second runtime in the process, and torch's streams would not be
    # valid in this library's (its launches would fail).
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    lay_p = ctypes.POINTER(ZeroLayout)
    hp_p = ctypes.POINTER(_HParams)
    L.zero_abi_version.argtypes = []
    L.zero_abi_version.restype = i32
    L.zero_status_string.argtypes = [ctypes.c_int]
    L.zero_status_string.restype = ctypes.c_char_p
    L.zero_flatten_layout.argtypes = [vp, i64, i32, i64, vp, lay_p]
    L.zero_flatten_layout.restype = ctypes.c_int
    L.zero_shard_segments.argtypes = [lay_p, vp, i64, i32, vp, i64, ctypes.POINTER(i64)]
    L.zero_shard_segments.restype = ctypes.c_int
    L.zero_array_split_layout.argtypes = [i64, i32, vp, vp]
    L.zero_array_split_layout.restype = ctypes.c_int
    L.zero_dim0_layout.argtypes = [vp, vp, i64, i32, i64, vp, vp, lay_p]
    L.zero_dim0_layout.restype = ctypes.c_int
    L.zero_dim0_segments.argtypes = [lay_p, vp, vp, i64, i32, vp, i64, ctypes.POINTER(i64)]
    L.zero_dim0_segments.restype = ctypes.c_int
    L.zero_sumsq_workspace_bytes.argtypes = [i64]
    L.zero_sumsq_workspace_bytes.restype = i64
    L.zero_shard_reduce.argtypes = [vp, ctypes.c_int, i32, i64, i64, vp, i32, vp, vp, vp, i64,
                                    vp]
    L.zero_shard_reduce.restype = ctypes.c_int
    L.zero_shard_adamw.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, lay_p, i32, i64, i64,
                                   hp_p, vp, vp]
    L.zero_shard_adamw.restype = ctypes.c_int
    L.zero_shard_adamw_ex.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, lay_p, i32, i64, i64,
                                      hp_p, ctypes.POINTER(_StepControl), vp]
    L.zero_shard_adamw_ex.restype = ctypes.c_int
    L.zero_loss_scale_update.argtypes = [vp, vp, dbl, dbl, i32, vp]
    L.zero_loss_scale_update.restype = ctypes.c_int
    L.zero_shard_step.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, vp, vp, ctypes.c_int,
                                  lay_p, i32, i64, hp_p, vp, vp, vp, i64, vp]
    L.zero_shard_step.restype = ctypes.c_int
    L.zero_shard_step_noalloc.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, vp, vp,
                                          ctypes.c_int, lay_p, i32, i64, hp_p, vp, vp, vp]
    L.zero_shard_step_noalloc.restype = ctypes.c_int
    L.zero_step_consts_make.argtypes = [hp_p, ctypes.POINTER(ZeroStepConsts)]
    L.zero_step_consts_make.restype = ctypes.c_int
    L.zero_shard_step_dc.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, vp, vp, ctypes.c_int,
                                     lay_p, i32, i64, vp, vp, vp, vp, i64, vp]
    L.zero_shard_step_dc.restype = ctypes.c_int
    L.zero_shard_adamw_dc.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, lay_p, i32, i64, i64,
                                      vp, ctypes.POINTER(_StepControl), vp]
    L.zero_shard_adamw_dc.restype = ctypes.c_int
    L.zero_step_consts_select.argtypes = [vp, vp, i64, vp, vp]
    L.zero_step_consts_select.restype = ctypes.c_int
    L.zero_step_counter_advance.argtypes = [vp, vp, vp]
    L.zero_step_counter_advance.restype = ctypes.c_int
    piece_p = ctypes.POINTER(_Piece)
    L.zero_flat_gather.argtypes = [piece_p, i32, i64, i32, i64, i64, vp, vp]
    L.zero_flat_gather.restype = ctypes.c_int
    L.zero_flat_scatter.argtypes = [vp, i64, i64, piece_p, i32, i32, vp]
    L.zero_flat_scatter.restype = ctypes.c_int
    L.zero_reshard.argtypes = [ctypes.POINTER(vp), i32, i64, i64, i32, i32, i64, vp, vp]
    L.zero_reshard.restype = ctypes.c_int
    L.zero_q8_quantize.argtypes = [vp, ctypes.c_int, i64, vp, vp, vp]
    L.zero_q8_quantize.restype = ctypes.c_int
    L.zero_q8_dequantize.argtypes = [vp, vp, i64, vp, ctypes.c_int, vp]
    L.zero_q8_dequantize.restype = ctypes.c_int
    L.zero_shard_step_q8.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, lay_p, i32, i64,
                                     hp_p, vp, vp, vp, i64, vp]
    L.zero_shard_step_q8.restype = ctypes.c_int
    L.zero_shard_step_q8_dc.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, lay_p, i32,
                                        i64, vp, vp, vp, vp, i64, vp]
    L.zero_shard_step_q8_dc.restype = ctypes.c_int
    L.zero_model_state_bytes.argtypes = [dbl, dbl, i32, dbl, ctypes.POINTER(dbl)]
    L.zero_model_state_bytes.restype = ctypes.c_int
    L.zero_comm_bytes.argtypes = [dbl, dbl, i32, dbl, dbl, ctypes.POINTER(dbl)]
    L.zero_comm_bytes.restype = ctypes.c_int
    if L.zero_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH}: ABI version {L.zero_abi_version()} != {ABI_VERSION}")
    return L


_lib = _load()


def _check(status: int, what: str):
    if status == ZERO_OK:
        return
    if status in (ZERO_EINVAL, ZERO_EALIAS, ZERO_ERANGE):
        raise ZeroValueError(status, what)
    raise ZeroError(status, what)


# ---------------------------------------------------------------------------
# argument marshalling


def _dtype_code(t, what: str, allow_fp32: bool = False) -> int:
    import torch
    if t.dtype in (torch.bfloat16,):
        return ZERO_BF16
    if t.dtype in (torch.float16,):
        return ZERO_FP16
    if allow_fp32 and t.dtype == torch.float32:
        return ZERO_FP32
    want = "bfloat16, float16 or float32" if allow_fp32 else "16-bit (bfloat16 or float16)"
    raise TypeError(f"{what}: {want} tensor expected, got {t.dtype}")


def _dev_ptr(t, what: str, dtype=None):
    """Device address of a CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if not getattr(t, "is_cuda", False):
        raise TypeError(f"{what}: a GPU tensor is required")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what}: {dtype} expected, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _buf(t, what: str, need: int, dtype=None, device=None):
    """Device address of a contiguous CUDA tensor of at least `need` elements
    (None -> NULL) on `device`.  The kernels take plain pointers and sizes,
    so this is where a tensor too short for the sizes passed beside it, a
    strided or expanded view, or a tensor on another GPU is refused --
    before anything is launched."""
    if t is None:
        return None
    p = _dev_ptr(t, what, dtype)
    if device is not None and t.device != device:
        raise ValueError(f"{what}: on {t.device}, the call's tensors are on {device}")
    if not t.is_contiguous():
        raise TypeError(f"{what}: a contiguous tensor is required")
    if t.numel() < need:
        raise ValueError(f"{what}: {need} elements needed, the tensor holds {t.numel()}")
    return p


def _rows_need(n_rows: int, ld: int, length: int) -> int:
    """Elements spanned by n_rows rows of stride ld, length each."""
    return 0 if length <= 0 or n_rows < 1 else (n_rows - 1) * ld + length


def _rows(t, what: str, n_rows: int, ld: int, length: int, dtype=None, device=None):
    """Device address of n_rows rows of `length` elements, row k at element
    k * ld: a contiguous tensor spanning them, or a 2-D view [rows][cols]
    with row stride ld (a column range of a wider slab) holding them."""
    if t is None:
        return None
    p = _dev_ptr(t, what, dtype)
    if device is not None and t.device != device:
        raise ValueError(f"{what}: on {t.device}, the call's tensors are on {device}")
    need = _rows_need(n_rows, ld, length)
    if t.is_contiguous():
        if t.numel() < need:
            raise ValueError(f"{what}: {need} elements needed, the tensor holds {t.numel()}")
        return p
    if not (t.dim() == 2 and t.stride(1) == 1 and t.stride(0) == ld):
        raise TypeError(f"{what}: contiguous rows, or a 2-D view of row stride {ld}, required")
    if need and (t.shape[0] < n_rows or t.shape[1] < length):
        raise ValueError(f"{what}: {n_rows} rows of {length} elements needed, "
                         f"the view is {tuple(t.shape)}")
    return p


def zero_sumsq_workspace_bytes(length: int) -> int:
    """Bytes of device workspace a call over `length` elements that sums
    squares needs (8 bytes per 256 elements plus 34 KiB)."""
    n = _lib.zero_sumsq_workspace_bytes(int(length))
    if n < 0:
        raise ValueError(f"zero_sumsq_workspace_bytes: length {length} out of range")
    return n


def _torch_stream(stream, device):
    """The call's stream as a torch stream: the current one for None, a
    torch stream as given, a raw hipStream_t handle wrapped."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _workspace(sumsq, workspace, length: int, device, stream=None):
    """(pointer, bytes) of the sum's workspace: the caller's (checked for
    size) or a new one; (NULL, 0) without a sum.  A new one is allocated on
    the call's stream: it is freed when the call returns, and torch's
    allocator reuses a block only in the order of the stream it was
    allocated on, so the call's kernels finish with it first."""
    import torch
    if sumsq is None:
        return None, 0
    need = zero_sumsq_workspace_bytes(max(0, length))
    if workspace is None:
        with torch.cuda.stream(_torch_stream(stream, device)):
            workspace = torch.empty((need + 7) // 8, dtype=torch.float64, device=device)
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError(f"workspace: {need} bytes needed, the tensor holds {nbytes}")
    return _buf(workspace, "workspace", 0, device=device), nbytes


def _stream(stream, like):
    return ctypes.c_void_p(_torch_stream(stream, like.device).cuda_stream)


# ---------------------------------------------------------------------------
# entry points


def zero_array_split_layout(n: int, n_dp: int) -> Tuple[np.ndarray, np.ndarray]:
    """(starts, lens) of the n_dp pieces numpy.array_split cuts n elements into."""
    starts = np.zeros(max(n_dp, 0), dtype=np.int64)
    lens = np.zeros(max(n_dp, 0), dtype=np.int64)
    _check(_lib.zero_array_split_layout(int(n), int(n_dp), starts.ctypes.data_as(ctypes.c_void_p),
                                        lens.ctypes.data_as(ctypes.c_void_p)),
           "zero_array_split_layout")
    return starts, lens


def zero_flatten_layout(numels: Sequence[int], n_dp: int, align: int = 1
                        ) -> Tuple[ZeroLayout, np.ndarray]:
    """Flat layout of the parameter list and each parameter's flat offset."""
    nums = np.ascontiguousarray(numels, dtype=np.int64)
    offs = np.zeros(len(nums), dtype=np.int64)
    lay = ZeroLayout()
    _check(_lib.zero_flatten_layout(nums.ctypes.data_as(ctypes.c_void_p), len(nums), n_dp,
                                    align, offs.ctypes.data_as(ctypes.c_void_p),
                                    ctypes.byref(lay)), "zero_flatten_layout")
    return lay, offs


def zero_shard_segments(layout: ZeroLayout, numels: Sequence[int], rank: int
                        ) -> List[Tuple[int, int, int, int]]:
    """(tensor, tensor_off, shard_off, len) pieces of shard `rank`; tensor -1 is padding."""
    nums = np.ascontiguousarray(numels, dtype=np.int64)
    cnt = ctypes.c_int64(0)
    p = nums.ctypes.data_as(ctypes.c_void_p)
    _check(_lib.zero_shard_segments(ctypes.byref(layout), p, len(nums), rank, None, 0,
                                    ctypes.byref(cnt)), "zero_shard_segments")
    segs = (_Segment * max(cnt.value, 1))()
    _check(_lib.zero_shard_segments(ctypes.byref(layout), p, len(nums), rank, segs, cnt.value,
                                    ctypes.byref(cnt)), "zero_shard_segments")
    return [(s.tensor, s.tensor_off, s.shard_off, s.len) for s in segs[:cnt.value]]


def _shape_arrays(shapes):
    rows = np.ascontiguousarray([int(r) for r, _ in shapes], dtype=np.int64)
    cols = np.ascontiguousarray([int(c) for _, c in shapes], dtype=np.int64)
    return rows, cols


def zero_dim0_layout(shapes: Sequence[Tuple[int, int]], n_dp: int, align: int = 1
                     ) -> Tuple[ZeroLayout, np.ndarray, np.ndarray]:
    """Per-parameter dim-0 layout of tensors [(rows, cols), ...]: the layout,
    each tensor's packed offset and its chunk of rows per rank."""
    rows, cols = _shape_arrays(shapes)
    offs = np.zeros(len(shapes), dtype=np.int64)
    chunk = np.zeros(len(shapes), dtype=np.int64)
    lay = ZeroLayout()
    _check(_lib.zero_dim0_layout(rows.ctypes.data_as(ctypes.c_void_p),
                                 cols.ctypes.data_as(ctypes.c_void_p), len(shapes), n_dp, align,
                                 offs.ctypes.data_as(ctypes.c_void_p),
                                 chunk.ctypes.data_as(ctypes.c_void_p), ctypes.byref(lay)),
           "zero_dim0_layout")
    return lay, offs, chunk


def zero_dim0_segments(layout: ZeroLayout, shapes: Sequence[Tuple[int, int]], rank: int
                       ) -> List[Tuple[int, int, int, int]]:
    """(tensor, tensor_off, shard_off, len) pieces of rank's packed buffer."""
    rows, cols = _shape_arrays(shapes)
    r_p, c_p = rows.ctypes.data_as(ctypes.c_void_p), cols.ctypes.data_as(ctypes.c_void_p)
    cnt = ctypes.c_int64(0)
    _check(_lib.zero_dim0_segments(ctypes.byref(layout), r_p, c_p, len(shapes), rank, None, 0,
                                   ctypes.byref(cnt)), "zero_dim0_segments")
    segs = (_Segment * max(cnt.value, 1))()
    _check(_lib.zero_dim0_segments(ctypes.byref(layout), r_p, c_p, len(shapes), rank, segs,
                                   cnt.value, ctypes.byref(cnt)), "zero_dim0_segments")
    return [(g.tensor, g.tensor_off, g.shard_off, g.len) for g in segs[:cnt.value]]


def zero_shard_reduce(grads, n_contrib: int, ld: int, length: int, acc,
                      accumulate: bool = False, overflow=None, sumsq=None, stream=None,
                      workspace=None):
    """acc[:length] (+)= sum of n_contrib rows (bf16, fp16 or fp32) of stride ld
    starting at grads; with sumsq, the sum of acc^2 is added to it (a
    workspace tensor is allocated unless one of at least
    zero_sumsq_workspace_bytes(length) bytes is passed)."""
    import torch
    d = acc.device
    ws, ws_bytes = _workspace(sumsq, workspace, length, d, stream)
    _check(_lib.zero_shard_reduce(
        _rows(grads, "grads", n_contrib, ld, length, device=d),
        _dtype_code(grads, "grads", True), n_contrib, ld, length,
        _buf(acc, "acc", length, torch.float32), int(bool(accumulate)),
        _buf(overflow, "overflow", 1, torch.int32, d), _buf(sumsq, "sumsq", 1, torch.float64, d),
        ws, ws_bytes, _stream(stream, acc)), "zero_shard_reduce")


def zero_shard_adamw(acc, master, m, v, weight_full, layout: ZeroLayout, rank: int,
                     hp: AdamWHParams, shard_off: int = 0, length: Optional[int] = None,
                     skip=None, stream=None):
    """AdamW on master/m/v[:length] from the fp32 gradient acc, cast into the slot."""
    import torch
    if length is None:
        length = master.numel()
    hpc = hp._c()
    d = master.device
    _check(_lib.zero_shard_adamw(
        _buf(acc, "acc", length, torch.float32, d), _buf(master, "master", length, torch.float32),
        _buf(m, "m", length, torch.float32, d), _buf(v, "v", length, torch.float32, d),
        _buf(weight_full, "weight_full", _slot_end(layout, rank, shard_off, length), device=d),
        _dtype_code(weight_full, "weight_full"),
        ctypes.byref(layout), rank, shard_off, length, ctypes.byref(hpc),
        _buf(skip, "skip", 1, torch.int32, d), _stream(stream, master)), "zero_shard_adamw")


def zero_shard_adamw_ex(acc, master, m, v, weight_full, layout: ZeroLayout, rank: int,
                        hp: AdamWHParams, shard_off: int = 0, length: Optional[int] = None,
                        skip=None, sumsq=None, max_norm: float = 0.0, loss_scale=None,
                        stream=None):
    """zero_shard_adamw with controls: skip (int32 flag), clipping from the
    whole-model sum of squares (float64 scalar) to max_norm, and a dynamic
    loss scale (see new_loss_scale)."""
    import torch
    if length is None:
        length = master.numel()
    hpc = hp._c()
    d = master.device
    ctl = _StepControl(_buf(skip, "skip", 1, torch.int32, d),
                       _buf(sumsq, "sumsq", 1, torch.float64, d), float(max_norm),
                       _buf(loss_scale, "loss_scale", 2, torch.int32, d))
    _check(_lib.zero_shard_adamw_ex(
        _buf(acc, "acc", length, torch.float32, d), _buf(master, "master", length, torch.float32),
        _buf(m, "m", length, torch.float32, d), _buf(v, "v", length, torch.float32, d),
        _buf(weight_full, "weight_full", _slot_end(layout, rank, shard_off, length), device=d),
        _dtype_code(weight_full, "weight_full"),
        ctypes.byref(layout), rank, shard_off, length, ctypes.byref(hpc), ctypes.byref(ctl),
        _stream(stream, master)), "zero_shard_adamw_ex")


def new_loss_scale(scale: float = 65536.0, device="cuda"):
    """A device zero_loss_scale {float scale; int32 good_steps} as an int32[2] tensor."""
    import torch
    bits = int(np.array([scale], dtype=np.float32).view(np.int32)[0])
    return torch.tensor([bits, 0], dtype=torch.int32, device=device)


def read_loss_scale(t) -> Tuple[float, int]:
    h = t.detach().cpu().numpy().astype(np.int32)
    return float(h[:1].view(np.float32)[0]), int(h[1])


def zero_loss_scale_update(loss_scale, overflow, growth: float = 2.0, backoff: float = 0.5,
                           interval: int = 2000, stream=None):
    """One step of the device-resident dynamic loss scale."""
    import torch
    _check(_lib.zero_loss_scale_update(
        _buf(loss_scale, "loss_scale", 2, torch.int32),
        _buf(overflow, "overflow", 1, torch.int32, loss_scale.device),
        float(growth), float(backoff), int(interval), _stream(stream, loss_scale)),
        "zero_loss_scale_update")


def zero_shard_step(grads, ld: int, length: int, master, m, v, weight_full,
                    layout: ZeroLayout, rank: int, hp: AdamWHParams, shard_off: int = 0,
                    overflow=None, sumsq=None, stream=None, workspace=None):
    """Fused reduce of layout.n_dp rows + AdamW + cast into the weight slot
    (sumsq and workspace as for zero_shard_reduce)."""
    import torch
    hpc = hp._c()
    d = master.device
    ws, ws_bytes = _workspace(sumsq, workspace, length, d, stream)
    _check(_lib.zero_shard_step(
        _rows(grads, "grads", layout.n_dp, ld, length, device=d),
        _dtype_code(grads, "grads", True), ld, length,
        _buf(master, "master", length, torch.float32), _buf(m, "m", length, torch.float32, d),
        _buf(v, "v", length, torch.float32, d),
        _buf(weight_full, "weight_full", _slot_end(layout, rank, shard_off, length), device=d),
        _dtype_code(weight_full, "weight_full"), ctypes.byref(layout), rank, shard_off,
        ctypes.byref(hpc), _buf(overflow, "overflow", 1, torch.int32, d),
        _buf(sumsq, "sumsq", 1, torch.float64, d), ws, ws_bytes, _stream(stream, master)),
        "zero_shard_step")


ZERO_NOALLOC_MAX_LEN = 1 << 29


def zero_shard_step_noalloc(grads, ld: int, length: int, master, m, v, weight_full,
                            layout: ZeroLayout, rank: int, hp: AdamWHParams, shard_off: int = 0,
                            overflow=None, sumsq=None, stream=None):
    """zero_shard_step for callers that cannot allocate: the sum of squares
    goes through the library's own device scratch (no workspace argument,
    nothing allocated, here or in the library).  With sumsq, length is at
    most ZERO_NOALLOC_MAX_LEN; calls that sum squares on one GPU must not
    run concurrently (they share the scratch)."""
    import torch
    if sumsq is not None and length > ZERO_NOALLOC_MAX_LEN:
        raise ZeroValueError(ZERO_EINVAL, f"zero_shard_step_noalloc: length {length} is above "
                             f"ZERO_NOALLOC_MAX_LEN = {ZERO_NOALLOC_MAX_LEN} with a sum of "
                             "squares; split the range into several calls")
    hpc = hp._c()
    d = master.device
    _check(_lib.zero_shard_step_noalloc(
        _rows(grads, "grads", layout.n_dp, ld, length, device=d),
        _dtype_code(grads, "grads", True), ld, length,
        _buf(master, "master", length, torch.float32), _buf(m, "m", length, torch.float32, d),
        _buf(v, "v", length, torch.float32, d),
        _buf(weight_full, "weight_full", _slot_end(layout, rank, shard_off, length), device=d),
        _dtype_code(weight_full, "weight_full"), ctypes.byref(layout), rank, shard_off,
        ctypes.byref(hpc), _buf(overflow, "overflow", 1, torch.int32, d),
        _buf(sumsq, "sumsq", 1, torch.float64, d), _stream(stream, master)),
        "zero_shard_step_noalloc")


def zero_step_consts_make(hp: AdamWHParams) -> np.ndarray:
    """The step's constants (a zero_step_consts, 48 bytes) as a uint8 array,
    to be copied into a device buffer from new_step_consts() before the
    _dc calls (or a graph of them) run."""
    out = ZeroStepConsts()
    hpc = hp._c()
    _check(_lib.zero_step_consts_make(ctypes.byref(hpc), ctypes.byref(out)),
           "zero_step_consts_make")
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


def new_step_consts(device="cuda"):
    """A device buffer for one zero_step_consts (uint8[48])."""
    import torch
    return torch.zeros(ctypes.sizeof(ZeroStepConsts), dtype=torch.uint8, device=device)


def step_consts_table(hps, device="cuda"):
    """A device table of step constants, row k those of hps[k] (for the
    device counter, row k serves step k + 1): uint8[len(hps)][48]."""
    import torch
    rows = np.stack([zero_step_consts_make(hp) for hp in hps])
    return torch.from_numpy(rows).to(device)


def new_step_counter(t: int = 1, device="cuda"):
    """A device step counter (int64[1]) holding t."""
    import torch
    return torch.tensor([int(t)], dtype=torch.int64, device=device)


def zero_step_consts_select(consts, table, t, stream=None):
    """consts = table[*t - 1] on the device (all NaN when *t is outside the
    table's rows)."""
    import torch
    d = consts.device
    if table.dim() != 2 or table.shape[1] != ctypes.sizeof(ZeroStepConsts):
        raise ValueError("zero_step_consts_select: table must be uint8[count][48]")
    count = table.shape[0]
    _check(_lib.zero_step_consts_select(
        _consts(consts, d), _buf(table, "table", count * ctypes.sizeof(ZeroStepConsts),
                                 torch.uint8, d), count,
        _buf(t, "t", 1, torch.int64, d), _stream(stream, consts)), "zero_step_consts_select")


def zero_step_counter_advance(t, skip=None, stream=None):
    """*t += 1 on the device unless skip (int32 flag) is non-zero."""
    import torch
    _check(_lib.zero_step_counter_advance(
        _buf(t, "t", 1, torch.int64), _buf(skip, "skip", 1, torch.int32, t.device),
        _stream(stream, t)), "zero_step_counter_advance")


def _consts(consts, device):
    import torch
    return _buf(consts, "consts", ctypes.sizeof(ZeroStepConsts), torch.uint8, device)


def zero_shard_step_dc(grads, ld: int, length: int, master, m, v, weight_full,
                       layout: ZeroLayout, rank: int, consts, shard_off: int = 0,
                       overflow=None, sumsq=None, stream=None, workspace=None):
    """zero_shard_step with the constants read from the device buffer consts
    (see zero_step_consts_make) when the kernels run."""
    import torch
    d = master.device
    ws, ws_bytes = _workspace(sumsq, workspace, length, d, stream)
    _check(_lib.zero_shard_step_dc(
        _rows(grads, "grads", layout.n_dp, ld, length, device=d),
        _dtype_code(grads, "grads", True), ld, length,
        _buf(master, "master", length, torch.float32), _buf(m, "m", length, torch.float32, d),
        _buf(v, "v", length, torch.float32, d),
        _buf(weight_full, "weight_full", _slot_end(layout, rank, shard_off, length), device=d),
        _dtype_code(weight_full, "weight_full"), ctypes.byref(layout), rank, shard_off,
        _consts(consts, d), _buf(overflow, "overflow", 1, torch.int32, d),
        _buf(sumsq, "sumsq", 1, torch.float64, d), ws, ws_bytes, _stream(stream, master)),
        "zero_shard_step_dc")


def zero_shard_adamw_dc(acc, master, m, v, weight_full, layout: ZeroLayout, rank: int, consts,
                        shard_off: int = 0, length: Optional[int] = None, skip=None,
                        sumsq=None, max_norm: float = 0.0, loss_scale=None, stream=None):
    """zero_shard_adamw_ex with the constants read from the device buffer
    consts when the kernels run."""
    import torch
    if length is None:
        length = master.numel()
    d = master.device
    ctl = _StepControl(_buf(skip, "skip", 1, torch.int32, d),
                       _buf(sumsq, "sumsq", 1, torch.float64, d), float(max_norm),
                       _buf(loss_scale, "loss_scale", 2, torch.int32, d))
    _check(_lib.zero_shard_adamw_dc(
        _buf(acc, "acc", length, torch.float32, d), _buf(master, "master", length, torch.float32),
        _buf(m, "m", length, torch.float32, d), _buf(v, "v", length, torch.float32, d),
        _buf(weight_full, "weight_full", _slot_end(layout, rank, shard_off, length), device=d),
        _dtype_code(weight_full, "weight_full"), ctypes.byref(layout), rank, shard_off, length,
        _consts(consts, d), ctypes.byref(ctl), _stream(stream, master)), "zero_shard_adamw_dc")


def _slot_end(layout: ZeroLayout, rank: int, shard_off: int, length: int) -> int:
    """One past the last element of the weight buffer a call writes."""
    return 0 if length <= 0 else rank * layout.shard + shard_off + length


def _elem_bytes(ts, what: str) -> int:
    sizes = {t.element_size() for t in ts}
    if len(sizes) != 1:
        raise TypeError(f"{what}: all tensors must have one element size, got {sorted(sizes)}")
    for t in ts:
        if not t.is_contiguous():
            raise TypeError(f"{what}: contiguous tensors expected")
    return sizes.pop()


def _pieces(pieces, what: str, device):
    arr = (_Piece * max(1, len(pieces)))()
    for i, (t, off) in enumerate(pieces):
        arr[i] = _Piece(_buf(t, what, 0, device=device), int(off), t.numel())
    return arr


def zero_flat_gather(pieces, n: int, begin: int, dst, stream=None):
    """dst[j] = flat[begin + j] for j < dst.numel(), from pieces
    [(tensor, flat_off), ...]; zeros where no piece holds the index or it is
    >= n.  Bitwise, for 2- or 4-byte elements."""
    eb = _elem_bytes([dst] + [t for t, _ in pieces], "zero_flat_gather")
    _check(_lib.zero_flat_gather(_pieces(pieces, "piece", dst.device), len(pieces), n, eb, begin,
                                 dst.numel(), _dev_ptr(dst, "dst"), _stream(stream, dst)),
           "zero_flat_gather")


def zero_flat_scatter(src, begin: int, pieces, stream=None):
    """Writes src (flat indices [begin, begin + src.numel())) into the pieces
    [(tensor, flat_off), ...] where they hold those indices."""
    eb = _elem_bytes([src] + [t for t, _ in pieces], "zero_flat_scatter")
    _check(_lib.zero_flat_scatter(_dev_ptr(src, "src"), begin, src.numel(),
                                  _pieces(pieces, "piece", src.device), len(pieces), eb,
                                  _stream(stream, src)), "zero_flat_scatter")


def zero_reshard(src_shards, n: int, dst_rank: int, dst, stream=None):
    """dst (one shard of dst.numel() elements) = new rank dst_rank's shard of
    the flat vector of n elements held as the equal old shards src_shards."""
    eb = _elem_bytes([dst] + list(src_shards), "zero_reshard")
    sizes = {t.numel() for t in src_shards}
    if len(sizes) != 1:
        raise ValueError("zero_reshard: the old shards must have one size")
    ptrs = (ctypes.c_void_p * len(src_shards))(*[_buf(t, "src_shard", 0, device=dst.device).value
                                                 for t in src_shards])
    _check(_lib.zero_reshard(ptrs, len(src_shards), sizes.pop(), n, eb, dst_rank, dst.numel(),
                             _dev_ptr(dst, "dst"), _stream(stream, dst)), "zero_reshard")


def q8_blocks(length: int) -> int:
    """Scales of a quantized vector of `length` elements."""
    return (length + ZERO_Q8_BLOCK - 1) // ZERO_Q8_BLOCK


def zero_q8_quantize(x, q, scales, stream=None):
    """Blockwise int8 codes (int8 tensor q) and fp32 scales of x (bf16,
    fp16 or fp32), one scale per ZERO_Q8_BLOCK elements."""
    import torch
    n, d = x.numel(), x.device
    _check(_lib.zero_q8_quantize(_buf(x, "x", n), _dtype_code(x, "x", True), n,
                                 _buf(q, "q", n, torch.int8, d),
                                 _buf(scales, "scales", q8_blocks(n), torch.float32, d),
                                 _stream(stream, x)), "zero_q8_quantize")


def zero_q8_dequantize(q, scales, y, stream=None):
    """y = codes x block scale, stored in y's dtype (bf16, fp16 or fp32)."""
    import torch
    n, d = q.numel(), q.device
    _check(_lib.zero_q8_dequantize(_buf(q, "q", n, torch.int8),
                                   _buf(scales, "scales", q8_blocks(n), torch.float32, d), n,
                                   _buf(y, "y", n, device=d), _dtype_code(y, "y", True),
                                   _stream(stream, q)), "zero_q8_dequantize")


def zero_shard_step_q8(gq, gscales, ld: int, sld: int, length: int, master, m, v, wq_full,
                       wscales_full, layout: ZeroLayout, rank: int, hp: AdamWHParams,
                       shard_off: int = 0, overflow=None, sumsq=None, stream=None,
                       workspace=None):
    """Fused step with 8-bit rows in (codes gq, scales gscales) and 8-bit
    weights out (wq_full, wscales_full: the all-gather buffer); sumsq and
    workspace as for zero_shard_reduce."""
    import torch
    hpc = hp._c()
    d = master.device
    ws, ws_bytes = _workspace(sumsq, workspace, length, d, stream)
    nb = q8_blocks(length)
    end = _slot_end(layout, rank, shard_off, length)
    _check(_lib.zero_shard_step_q8(
        _rows(gq, "gq", layout.n_dp, ld, length, torch.int8, d),
        _rows(gscales, "gscales", layout.n_dp, sld, nb, torch.float32, d), ld, sld,
        length, _buf(master, "master", length, torch.float32), _buf(m, "m", length, torch.float32, d),
        _buf(v, "v", length, torch.float32, d), _buf(wq_full, "wq_full", end, torch.int8, d),
        _buf(wscales_full, "wscales_full",
             0 if length <= 0 else (end - length) // ZERO_Q8_BLOCK + nb, torch.float32, d),
        ctypes.byref(layout), rank, shard_off, ctypes.byref(hpc),
        _buf(overflow, "overflow", 1, torch.int32, d), _buf(sumsq, "sumsq", 1, torch.float64, d),
        ws, ws_bytes, _stream(stream, master)), "zero_shard_step_q8")


def zero_shard_step_q8_dc(gq, gscales, ld: int, sld: int, length: int, master, m, v, wq_full,
                          wscales_full, layout: ZeroLayout, rank: int, consts,
                          shard_off: int = 0, overflow=None, sumsq=None, stream=None,
                          workspace=None):
    """zero_shard_step_q8 with the constants read from the device buffer
    consts (see zero_step_consts_make) when the kernels run."""
    import torch
    d = master.device
    ws, ws_bytes = _workspace(sumsq, workspace, length, d, stream)
    nb = q8_blocks(length)
    end = _slot_end(layout, rank, shard_off, length)
    _check(_lib.zero_shard_step_q8_dc(
        _rows(gq, "gq", layout.n_dp, ld, length, torch.int8, d),
        _rows(gscales, "gscales", layout.n_dp, sld, nb, torch.float32, d), ld, sld,
        length, _buf(master, "master", length, torch.float32), _buf(m, "m", length, torch.float32, d),
        _buf(v, "v", length, torch.float32, d), _buf(wq_full, "wq_full", end, torch.int8, d),
        _buf(wscales_full, "wscales_full",
             0 if length <= 0 else (end - length) // ZERO_Q8_BLOCK + nb, torch.float32, d),
        ctypes.byref(layout), rank, shard_off, _consts(consts, d),
        _buf(overflow, "overflow", 1, torch.int32, d), _buf(sumsq, "sumsq", 1, torch.float64, d),
        ws, ws_bytes, _stream(stream, master)), "zero_shard_step_q8_dc")


def zero_adam_step(grads, w_shards, m_shards, v_shards, t: int, lr: float = 1e-3,
                   b1: float = 0.9, b2: float = 0.999, eps: float = 1e-8,
                   weight_decay: float = 0.0, stream=None):
    """The functional form of one sharded Adam step for n_dp ranks simulated
    on one GPU ("ZeRO and FSDP", "A sharded Adam step").

    grads[r]: rank r's full local gradient (1-D, length n; fp32, bf16 or
    fp16); w_shards[r], m_shards[r], v_shards[r]: rank r's fp32 piece of
    numpy.array_split(range(n), n_dp).  Returns (full_w, w_shards, m_shards,
    v_shards): full_w[r] is rank r's fp32 copy of the whole updated weight
    vector (the all-gather's result), the shard lists are new tensors, and
    no input is modified.  Rank r's gradient is the average over ranks of
    its piece (the reduce-scatter's arithmetic: a left-to-right fp32 sum
    times fl(1/n_dp)); Adam with bias correction from t = 1 (AdamW with
    weight_decay > 0).  Every step runs in the library's kernels: the flat
    copies build the gradient slab, clone the shards and gather the full
    weights; the reduce and AdamW kernels update each rank's piece.  Every
    tensor it allocates -- the temporaries and the results -- belongs to the
    call's stream, where all its work runs, so the temporaries freed on
    return are reused only after that work."""
    import torch
    n_dp = len(grads)
    if n_dp < 1 or not (len(w_shards) == len(m_shards) == len(v_shards) == n_dp):
        raise ValueError("zero_adam_step: one gradient and one shard of each state per rank")
    n = grads[0].numel()
    if any(g.numel() != n or g.dtype != grads[0].dtype for g in grads):
        raise ValueError("zero_adam_step: every rank's gradient is one vector of n elements")
    starts, lens = (a.tolist() for a in zero_array_split_layout(n, n_dp))
    for shards in (w_shards, m_shards, v_shards):
        for r, x in enumerate(shards):
            if x.numel() != lens[r] or x.dtype != torch.float32:
                raise ValueError(f"zero_adam_step: shard {r} must be fp32 of {lens[r]} elements")
    dev = grads[0].device
    with torch.cuda.stream(_torch_stream(stream, dev)):
        return _adam_step_on(grads, w_shards, m_shards, v_shards, t, lr, b1, b2, eps,
                             weight_decay, n_dp, n, lens, starts, dev)


def _adam_step_on(grads, w_shards, m_shards, v_shards, t, lr, b1, b2, eps, weight_decay, n_dp,
                  n, lens, starts, dev):
    """zero_adam_step's work, on the current stream."""
    import torch
    stream = None
    # the contributions as one [n_dp][n] slab (row k = rank k's gradient)
    slab = torch.empty(n_dp * n, dtype=grads[0].dtype, device=dev)
    zero_flat_gather([(g.reshape(-1), k * n) for k, g in enumerate(grads)], n_dp * n, 0, slab,
                     stream=stream)

    def clone(x):
        y = torch.empty_like(x)
        zero_flat_gather([(x.reshape(-1), 0)], x.numel(), 0, y, stream=stream)
        return y

    new_w = [clone(x) for x in w_shards]
    new_m = [clone(x) for x in m_shards]
    new_v = [clone(x) for x in v_shards]
    whole, _ = zero_flatten_layout([n], 1)         # one slot: the 16-bit weights of all n
    w16 = torch.empty(n, dtype=torch.bfloat16, device=dev)
    hp = AdamWHParams(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=weight_decay,
                      grad_scale=1.0 / n_dp, step=t)
    for r in range(n_dp):
        if lens[r] == 0:
            continue
        acc = torch.empty(lens[r], dtype=torch.float32, device=dev)
        zero_shard_reduce(slab[starts[r]:], n_dp, n, lens[r], acc, stream=stream)
        zero_shard_adamw(acc, new_w[r], new_m[r], new_v[r], w16, whole, 0, hp,
                         shard_off=starts[r], length=lens[r], stream=stream)
    pieces = [(x, s0) for x, s0 in zip(new_w, starts) if x.numel() > 0]
    full_w = []
    for _ in range(n_dp):  # the all-gather: every rank receives the whole vector
        f = torch.empty(n, dtype=torch.float32, device=dev)
        zero_flat_gather(pieces, n, 0, f, stream=stream)
        full_w.append(f)
    return full_w, new_w, new_m, new_v


def zero_model_state_bytes(n: float, n_dp: float, stage: int, k: float = 12) -> float:
    out = ctypes.c_double()
    _check(_lib.zero_model_state_bytes(n, n_dp, stage, k, ctypes.byref(out)),
           "zero_model_state_bytes")
    return out.value


def zero_comm_bytes(n: float, n_dp: float, stage: int, param_bytes: float = 2,
                    grad_bytes: float = 2) -> float:
    out = ctypes.c_double()
    _check(_lib.zero_comm_bytes(n, n_dp, stage, param_bytes, grad_bytes, ctypes.byref(out)),
           "zero_comm_bytes")
    return out.value


def library_path() -> str:
    return LIB_PATH


__all__ = ["zero_flatten_layout", "zero_shard_segments", "zero_dim0_layout", "zero_dim0_segments", "zero_shard_reduce",
           "zero_shard_adamw", "zero_shard_adamw_ex", "zero_loss_scale_update",
           "new_loss_scale", "read_loss_scale", "zero_shard_step", "zero_flat_gather",
           "zero_flat_scatter", "zero_reshard", "zero_q8_quantize", "zero_q8_dequantize",
           "zero_shard_step_q8", "zero_sumsq_workspace_bytes", "q8_blocks", "ZERO_Q8_BLOCK", "zero_model_state_bytes", "zero_comm_bytes",
           "zero_adam_step", "AdamWHParams", "ZeroLayout", "ZeroError", "ZeroValueError", "ZERO_BF16", "ZERO_FP16", "ZERO_FP32", "library_path"]
