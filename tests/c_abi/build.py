"""Build the C-only check of the library's C ABI (tests/c_abi/step_check):
plain C against include/zero_shard.h and the HIP runtime API, linked with
the library and the C oracle (test infrastructure), found at run time
relative to the binary."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "step_check")


def build(verbose: bool = False) -> str:
    lib_dir = os.path.join(ROOT, "zero_sharded_mixed_flatten_amd", "lib")
    ora_dir = os.path.join(ROOT, "oracle")
    rpath = "$ORIGIN/../../zero_sharded_mixed_flatten_amd/lib:$ORIGIN/../../oracle:/opt/rocm/lib"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", ora_dir,
           "-o", EXE + ".tmp", os.path.join(HERE, "step_check.c"),
           "-L", lib_dir, "-lzero_shard", "-L", ora_dir, "-loracle_zero",
           "-L/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{rpath}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
