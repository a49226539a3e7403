"""Build the host C/C++ code of this repository with AddressSanitizer and
UndefinedBehaviorSanitizer, for tests/test_sanitizers.py (CPU only):

  liboracle_zero_san.so  oracle/oracle_zero.c            (gcc)
  libsynth_san.so        synth/synth_cpu.c               (gcc, pthreads)
  liblayout_san.so       the library's host-only layout.cpp (g++)

Same numerics flags as the regular builds (-ffp-contract=off, no fast-math),
-O1 -g for readable reports, and every sanitizer finding fatal
(-fno-sanitize-recover=all).  No GPU code is built here."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
       "-Wall"]
ORACLE = os.path.join(HERE, "liboracle_zero_san.so")
SYNTH = os.path.join(HERE, "libsynth_san.so")
LAYOUT = os.path.join(HERE, "liblayout_san.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False):
    _run(["gcc", "-std=c11"] + SAN + ["-o", ORACLE, os.path.join(ROOT, "oracle", "oracle_zero.c"),
                                      "-lm"], verbose)
    _run(["gcc", "-std=c11", "-pthread"] + SAN +
         ["-o", SYNTH, os.path.join(ROOT, "synth", "synth_cpu.c"), "-lm"], verbose)
    _run(["g++", "-std=c++17"] + SAN +
         ["-I", os.path.join(ROOT, "include"), "-o", LAYOUT,
          os.path.join(ROOT, "zero_sharded_mixed_flatten_amd", "csrc", "layout.cpp")], verbose)
    return ORACLE, SYNTH, LAYOUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
