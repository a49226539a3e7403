"""The binding's ctypes structures have the C header's layout: a small C
program built against include/zero_shard.h prints sizeof and the offset of
every field the binding declares (a field the header does not have fails
to compile), and each must equal what ctypes computes.  The device-resident
loss scale, which the binding handles as an int32[2] tensor, is checked the
same way."""
import ctypes
import json
import os
import subprocess
import tempfile

import zero_sharded_mixed_flatten_amd as zs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

STRUCTS = {
    "zero_layout": zs.ZeroLayout,
    "zero_adamw_hparams": zs._HParams,
    "zero_segment": zs._Segment,
    "zero_step_control": zs._StepControl,
    "zero_piece": zs._Piece,
    "zero_step_consts": zs.ZeroStepConsts,
}


def _c_layout(fields):
    """{struct: [sizeof, {field: offsetof}]} as the C compiler lays them out."""
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "zero_shard.h"',
             "int main(void) {", '    printf("{");']
    first = True
    for name, flds in fields.items():
        sep = "" if first else ","
        first = False
        lines.append(f'    printf("{sep}\\"{name}\\": [%zu, {{", sizeof({name}));')
        for i, f in enumerate(flds):
            s2 = "" if i == 0 else ","
            lines.append(f'    printf("{s2}\\"{f}\\": %zu", offsetof({name}, {f}));')
        lines.append('    printf("}]");')
    lines += ['    printf("}\\n");', "    return 0;", "}"]
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "layout.c"), os.path.join(d, "layout")
        with open(src, "w") as f:
            f.write("\n".join(lines))
        subprocess.run(["gcc", "-std=c11", "-Wall", "-I", os.path.join(ROOT, "include"), "-o", exe,
                        src], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    return json.loads(out)


def test_ctypes_structures_match_the_header():
    fields = {name: [f for f, _ in cls._fields_] for name, cls in STRUCTS.items()}
    fields["zero_loss_scale"] = ["scale", "good_steps"]
    got = _c_layout(fields)
    for name, cls in STRUCTS.items():
        size, offs = got[name]
        assert size == ctypes.sizeof(cls), name
        for f, _ in cls._fields_:
            assert offs[f] == getattr(cls, f).offset, f"{name}.{f}"
    # the binding's int32[2] loss scale: the scale's bits, then the count
    assert got["zero_loss_scale"] == [8, {"scale": 0, "good_steps": 4}]
    assert ctypes.sizeof(zs.ZeroStepConsts) == 48
