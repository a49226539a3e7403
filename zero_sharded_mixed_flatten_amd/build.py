"""Build libzero_shard.so in-tree for gfx950 with hipcc.

Flags that the library's numerics rely on:
  -ffp-contract=off      no fused multiply-add anywhere (host constants too)
  no -ffast-math         HIP's default correctly rounded fp32 division and
                         square root, denormals kept
  -packed-fp32-ops off   packed fp32 instructions are never emitted
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIB_DIR, "libzero_shard.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("zero_shard.hip", "quant8.hip", "flat_copy.hip", "layout.cpp")]

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fPIC", "-shared", "-Wall", "-fvisibility=hidden"]


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    # only the entry points of include/zero_shard.h are exported
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"),
                             "-o", LIB + ".tmp"] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError("hipcc failed building libzero_shard.so")
    if verbose and err.strip():
        print(err, flush=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
