"""bench.py's same-mix ceiling kernel issues exactly the memory
instructions of the fused step it stands for (CPU): compiled for gfx950,
each instance (1, 8, 64 rows) holds n_dp 8-byte row loads, three 16-byte
state loads, three 16-byte state stores and one 8-byte slot store, with the
step's cache policies (non-temporal loads, non-temporal device-scope
stores).  The
state goes back unchanged, so its stores cannot be told from no stores by
the data; a compiler that treated them as no-ops (it once did, and the
kernel then reported 160 % of peak) is caught here."""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_ceiling_kernel_keeps_every_load_and_store():
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "--offload-device-only", "-S",
                        os.path.join(ROOT, "calibration", "stream_mix.hip"), "-o", out],
                       check=True, capture_output=True)
        lines = open(out).read().split("\n")
    seen = {}
    cur = None
    for line in lines:
        m = re.match(r"^(_Z\S*mix_kernelILi(\d+)E\S*):", line)
        if m:
            cur = int(m.group(2))
            seen[cur] = {"ld8": 0, "ld16": 0, "st16": 0, "st8": 0}
            continue
        if line.startswith(".Lfunc_end"):
            cur = None
        if cur is None:
            continue
        t = line.split()
        if not t:
            continue
        op = t[0]
        key = {"global_load_dwordx2": "ld8", "global_load_dwordx4": "ld16",
               "global_store_dwordx4": "st16", "global_store_dwordx2": "st8"}.get(op)
        if key:
            seen[cur][key] += 1
            pol = set(t[1:])
            assert ({"nt", "sc1"} <= pol) if key.startswith("st") else ("nt" in pol), line
    assert sorted(seen) == [1, 8, 64]
    for n_dp, c in seen.items():
        assert c == {"ld8": n_dp, "ld16": 3, "st16": 3, "st8": 1}, (n_dp, c)
