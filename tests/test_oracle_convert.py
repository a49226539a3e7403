"""The oracle's 16-bit conversions against library routines, exhaustively.

The widenings bf16 -> fp32 and fp16 -> fp32 are exact; the narrowings
fp32 -> bf16 and fp32 -> fp16 round to nearest, ties to even (the cast of
the updated master into the 16-bit weight slot, "ZeRO and FSDP", "The idea,
one stage at a time").  NaNs are compared by class only.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.util import same_or_both_nan16

ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_bf16_widen_all_patterns():
    ours = oracle.bf16_to_f32(ALL16).view(np.uint32)
    ref = torch.from_numpy(ALL16.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(ours, ref.view(np.uint32))


def test_f16_widen_all_patterns():
    ours = oracle.f16_to_f32(ALL16)
    ref = ALL16.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours.view(np.uint32)[~nan], ref.view(np.uint32)[~nan])


CHUNK = 1 << 22


def _chunks():
    base = np.arange(CHUNK, dtype=np.uint32)
    for c in range(0, 1 << 32, CHUNK):
        yield (base + np.uint32(c)).view(np.float32)


def _check(ours, ref, x, expmask, mantmask):
    if np.array_equal(ours, ref):
        return
    ok = same_or_both_nan16(ours, ref, expmask, mantmask)
    assert ok.all(), f"first mismatch at fp32 pattern {x.view(np.uint32)[~ok][0]:#x}"


def test_bf16_round_all_fp32_patterns():
    for x in _chunks():
        ours = oracle.f32_to_bf16(x)
        ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        _check(ours, ref, x, 0x7F80, 0x007F)


def test_f16_round_all_fp32_patterns():
    for x in _chunks():
        ours = oracle.f32_to_f16(x)
        ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
        _check(ours, ref, x, 0x7C00, 0x03FF)


@pytest.mark.parametrize("x,bits", [(1.0, 0x3F80), (-2.0, 0xC000), (np.inf, 0x7F80),
                                    (-0.0, 0x8000), (3.4028235e38, 0x7F80)])
def test_bf16_round_special_values(x, bits):
    assert oracle.f32_to_bf16(np.array([x], dtype=np.float32))[0] == bits
