"""Build the input generator: libsynth.so (gcc, host) and libsynth_gpu.so
(hipcc, gfx950).  Both compile synth_core.h with -ffp-contract=off so the
two builds draw identical values."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_CPU = os.path.join(HERE, "libsynth.so")
LIB_GPU = os.path.join(HERE, "libsynth_gpu.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False):
    _run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall",
          "-fPIC", "-shared", "-pthread", "-o", LIB_CPU + ".tmp",
          os.path.join(HERE, "synth_cpu.c"), "-lm"], verbose)
    os.replace(LIB_CPU + ".tmp", LIB_CPU)
    _run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fPIC", "-shared", "-o", LIB_GPU + ".tmp",
          os.path.join(HERE, "synth_gpu.hip")], verbose)
    os.replace(LIB_GPU + ".tmp", LIB_GPU)
    return LIB_CPU, LIB_GPU


if __name__ == "__main__":
    build(verbose=True)
