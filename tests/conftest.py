"""Shared pytest set-up: the repository root on sys.path, the `gpu` marker,
and the host-side libraries built on first use when nothing is built yet."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _ensure_built():
    import oracle
    import synth
    if not os.path.exists(oracle.LIB_PATH):
        from oracle import build as ob
        ob.build()
    if not os.path.exists(synth.LIB_CPU):
        from synth import build as sb
        sb.build()


_ensure_built()


@pytest.fixture(scope="session")
def cuda_device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)
