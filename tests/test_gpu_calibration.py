"""bench.py's same-mix ceiling kernel (calibration/stream_mix.hip) reads
what it stands for and writes the right places: the slot holds the XOR of
every row's 16-bit words, nothing around the slot is touched, and the state
comes back bit for bit.  (The state's stores write what was loaded, so
their presence is checked on the compiled kernel instead, in
tests/test_calibration_isa.py.)"""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    lib = ctypes.CDLL(os.path.join(ROOT, "calibration", "libstream_mix.so"))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.stream_mix.argtypes = [vp, i32, i64, i64, vp, vp, vp, vp, i32, vp]
    lib.stream_mix.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("n_dp", [1, 8, 64])
def test_stream_mix_moves_every_byte(n_dp):
    lib = _lib()
    rng = np.random.default_rng(n_dp)
    length, ld, pad = 65_536 + 1024, 65_536 + 2048, 512
    rows = rng.integers(0, 1 << 16, size=(n_dp, ld), dtype=np.uint16)
    state = [rng.standard_normal(length).astype(np.float32) for _ in range(3)]
    d_rows = torch.from_numpy(rows.view(np.int16)).cuda()
    d_state = [torch.from_numpy(s).cuda() for s in state]
    slot = torch.full((length + 2 * pad,), 0x5A5A, dtype=torch.int16, device="cuda")
    st = torch.cuda.current_stream()
    rc = lib.stream_mix(d_rows.data_ptr(), n_dp, ld, length, *(s.data_ptr() for s in d_state),
                        slot[pad:].data_ptr(), 7, ctypes.c_void_p(st.cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    for got, want in zip(d_state, state):
        assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))
    x = np.bitwise_xor.reduce(rows[:, :length], axis=0)
    got = slot.cpu().numpy().view(np.uint16)
    assert np.array_equal(got[pad:pad + length], x)
    assert np.all(got[:pad] == 0x5A5A) and np.all(got[pad + length:] == 0x5A5A)
    # a refused shape is a status, not a launch
    assert lib.stream_mix(d_rows.data_ptr(), 3, ld, length, *(s.data_ptr() for s in d_state),
                          slot[pad:].data_ptr(), 7, None) == 1
    assert lib.stream_mix(d_rows.data_ptr(), n_dp, ld, length - 2,
                          *(s.data_ptr() for s in d_state), slot[pad:].data_ptr(), 7, None) == 1
