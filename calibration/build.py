"""Build libstream_mix.so (bench.py's same-mix ceiling kernel) for gfx950."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libstream_mix.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fPIC", "-shared", "-Wall", "-fvisibility=hidden"]


def build(verbose: bool = False) -> str:
    cmd = [HIPCC] + FLAGS + ["-o", LIB + ".tmp", os.path.join(HERE, "stream_mix.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError("hipcc failed building libstream_mix.so")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
