"""The library's kernels keep the operation order the oracle defines (CPU):
every HIP source is compiled for gfx950 to AMD assembly and checked for the
instruction forms that would change rounding behind the source's back --
mixed-precision FMAs (v_fma_mix*, v_mad_mix*: one rounding to 16 bits where
the definition rounds to fp32 first) and packed fp32 arithmetic (disabled
for this hardware).  Plain v_fma_f32 is not listed: the correctly rounded
division and square root sequences use it internally; contraction of the
source's own multiply-adds is off in the build and the bitwise GPU tests
would show it.  The same scan requires that no kernel writes through the
scalar data cache: every store the compiler emits is a vector store.  And a
store written out in inline assembly with more than 64 bits of data must
itself provide the two wait states this chip needs before its data
registers may be overwritten (the compiler adds them after its own stores
only)."""
import functools
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_sharded_mixed_flatten_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = [os.path.join(CSRC, f) for f in ("zero_shard.hip", "quant8.hip", "flat_copy.hip")] + \
    [os.path.join(ROOT, "calibration", "stream_mix.hip")]

FORBIDDEN = [r"\bv_fma_mix", r"\bv_mad_mix", r"\bv_pk_fma_f32", r"\bv_pk_mul_f32",
             r"\bv_pk_add_f32"]
# the scalar data cache is never written -- no scalar stores or atomics, no
# write-back or discard of that cache: every store is a vector store
SCALAR_WRITES = [r"\bs_store", r"\bs_buffer_store", r"\bs_scratch_store", r"\bs_atomic",
                 r"\bs_buffer_atomic", r"\bs_dcache_wb", r"\bs_dcache_discard"]


@functools.lru_cache(maxsize=None)
def _asm(src):
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        # the library's own flags (build.py), device code only, as assembly
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17",
                        "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
                        "-packed-fp32-ops", "--offload-device-only", "-S",
                        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                        src, "-o", out],
                       check=True, capture_output=True)
        return open(out).read()


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES, ids=os.path.basename)
def test_no_rounding_changing_instructions(src):
    asm = _asm(src)
    kernels = len(re.findall(r"^\s*\.amdhsa_kernel\b", asm, flags=re.M))
    assert kernels > 0
    for pat in FORBIDDEN + SCALAR_WRITES:
        hits = re.findall(pat + r"[^\n]*", asm)
        assert not hits, f"{src}: {len(hits)} x {hits[0]}"


WIDE_STORE = re.compile(r"^\s*(global|buffer|flat)_store_dwordx[34]\b")
NOP = re.compile(r"^\s*s_nop\s+(\d+)")


def _inline_asm_blocks(asm):
    """the instruction lines of every inline-assembly block"""
    blocks, cur = [], None
    for line in asm.splitlines():
        if ";;#ASMSTART" in line:
            cur = []
        elif ";;#ASMEND" in line:
            blocks.append(cur)
            cur = None
        elif cur is not None and line.strip() and not line.strip().startswith(";"):
            cur.append(line)
    return blocks


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES, ids=os.path.basename)
def test_wide_inline_stores_carry_their_wait_states(src):
    blocks = _inline_asm_blocks(_asm(src))
    wide = 0
    for b in blocks:
        for i, line in enumerate(b):
            if WIDE_STORE.match(line):
                wide += 1
                nxt = b[i + 1] if i + 1 < len(b) else ""
                m = NOP.match(nxt)
                assert m and int(m.group(1)) >= 1, \
                    f"{os.path.basename(src)}: {line.strip()!r} followed by {nxt.strip()!r}"
    if os.path.basename(src) == "zero_shard.hip":
        assert wide > 0  # the fused step's state stores are written out
