"""The device build of the input generator draws exactly what the host
build draws (so oracle inputs regenerated on the host match the GPU's)."""
import numpy as np
import pytest
import torch

import synth
from synth import BF16, F16, F32, tag

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,sigma,thr,mul", [(F32, 0.02, 0, 1.0),
                                                (BF16, 1e-3, synth.outlier_threshold(0.01), 100.0),
                                                (F16, 65.536, 0, 1.0)])
def test_device_draws_equal_host_draws(kind, sigma, thr, mul):
    start, n = 123_456_789, 3_000_001
    tdt = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}[kind]
    d = torch.empty(n, dtype=tdt, device="cuda")
    synth.fill_device(d, kind, 0, tag(1, 2, 3, 4, 5), start, sigma, thr, mul)
    h = synth.fill_host(kind, 0, tag(1, 2, 3, 4, 5), start, n, sigma, thr, mul)
    got = d.cpu()
    got = got.numpy() if kind == F32 else got.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got.view(np.uint8), h.view(np.uint8))
