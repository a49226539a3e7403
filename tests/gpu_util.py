"""Helpers shared by the GPU tests: host <-> device transfers of raw 16-bit
patterns, parity comparisons at the stated bar, and seeded inputs."""
import numpy as np
import torch

import synth
from synth import BF16, F16, F32, tag
from synth.synth_const import BUF_GRAD, BUF_MASTER
from tests.util import rel_err, ulp16_diff

TDT = {0: torch.bfloat16, 1: torch.float16}  # ZERO_BF16, ZERO_FP16
SKIND = {0: BF16, 1: F16}


def dev16(a: np.ndarray, dt: int, device="cuda"):
    """uint16 host array -> 16-bit device tensor of dtype code dt."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(TDT[dt]).to(device)


def host16(t) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def devf(a: np.ndarray, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def hostf(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def is_nan16(h, dt):
    h = np.asarray(h, dtype=np.uint16)
    if dt == 0:
        return ((h & 0x7F80) == 0x7F80) & ((h & 0x7F) != 0)
    return ((h & 0x7C00) == 0x7C00) & ((h & 0x3FF) != 0)


def check_f32(gpu, ref, what, rel_tol=1e-6):
    """The fp32 bar: max |gpu - ref| / max(|ref|, 2^-126) <= rel_tol, NaN by
    class.  Returns the number of elements that are not bit-identical."""
    gpu = np.asarray(gpu, dtype=np.float32)
    ref = np.asarray(ref, dtype=np.float32)
    gn, rn = np.isnan(gpu), np.isnan(ref)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ"
    inf = np.isinf(ref)
    assert np.array_equal(gpu[inf], ref[inf]) and not np.isinf(gpu[~inf]).any(), \
        f"{what}: infinities differ"
    ok = ~rn & ~inf
    if ok.any():
        err = rel_err(gpu[ok], ref[ok]).max()
        assert err <= rel_tol, f"{what}: max rel err {err:.3g} > {rel_tol}"
    fin = ~rn
    return int(np.count_nonzero(gpu[fin].view(np.uint32) != ref[fin].view(np.uint32)))


def check_16(gpu, ref, dt, what, max_ulp=1):
    """The 16-bit bar: within max_ulp ulps, NaN by class.  Returns the number
    of elements that are not bit-identical."""
    gn, rn = is_nan16(gpu, dt), is_nan16(ref, dt)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ"
    ok = ~rn
    if ok.any():
        d = ulp16_diff(np.asarray(gpu)[ok], np.asarray(ref)[ok]).max()
        assert d <= max_ulp, f"{what}: {d} ulps > {max_ulp}"
    return int(np.count_nonzero(np.asarray(gpu)[ok] != np.asarray(ref)[ok]))


# ---- seeded inputs -------------------------------------------------------

def grad_tag(cfg, step, micro, k):
    return tag(BUF_GRAD, cfg, step, micro, k)


def master_tag(cfg):
    return tag(BUF_MASTER, cfg)


def host_rows(cfg, step, micro, n_rows, start, length, draw, pad_from=None):
    """[n_rows][length] uint16: rank k's flat gradient elements
    [start, start + length); flat indices >= pad_from are zero padding."""
    out = np.stack([synth.fill_host(draw.kind, 0, grad_tag(cfg, step, micro, k), start, length,
                                    draw.eff_sigma, draw.thr, draw.outlier_mul)
                    for k in range(n_rows)])
    if pad_from is not None and start + length > pad_from:
        out[:, max(0, pad_from - start):] = 0
    return out


def host_master(cfg, start, length, sigma=0.02, pad_from=None):
    w = synth.fill_host(F32, 0, master_tag(cfg), start, length, sigma)
    if pad_from is not None and start + length > pad_from:
        w[max(0, pad_from - start):] = 0
    return w


def gather_rows(cfg, step, micro, n_rows, flat_idx, draw):
    """[n_rows][len(idx)] uint16 for the given flat indices (for sampled checks)."""
    return np.stack([synth.gather_host(draw.kind, 0, grad_tag(cfg, step, micro, k), flat_idx,
                                       draw.eff_sigma, draw.thr, draw.outlier_mul)
                     for k in range(n_rows)])


def gather_master(cfg, flat_idx, sigma=0.02):
    return synth.gather_host(F32, 0, master_tag(cfg), flat_idx, sigma)


def device_rows(slab, cfg, step, micro, start, draw):
    """Fill the [n][ld] device slab's rows k with rank k's flat elements
    [start, start + ld) (the first `length` of them are used)."""
    n = slab.shape[0]
    for k in range(n):
        synth.fill_device(slab[k], draw.kind, 0, grad_tag(cfg, step, micro, k), start,
                          draw.eff_sigma, draw.thr, draw.outlier_mul)
    return slab


def device_master(w, cfg, start, sigma=0.02):
    return synth.fill_device(w, F32, 0, master_tag(cfg), start, sigma)
