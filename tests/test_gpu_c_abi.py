"""The C ABI from C alone, without Python or torch: tests/c_abi/step_check
(built by __graft_entry__.build()) allocates with hipMalloc, runs three
fused steps of one rank's shard through zero_shard_step and compares each
with the C oracle bit for bit -- master, moments and the whole weight
buffer."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "step_check")


def test_c_program_steps_bitwise():
    assert os.path.exists(EXE), "tests/c_abi/step_check is not built: run __graft_entry__.build()"
    print("\n[c-abi] running", EXE, flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"exit {r.returncode}: {r.stdout}{r.stderr}"
    assert "c-abi step ok" in r.stdout, r.stdout
