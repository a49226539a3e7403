"""The usage example in the README runs as printed: its first Python block
is executed on the GPU, then the weight slot it wrote is checked against the
round-to-nearest-even bf16 cast of the master it updated, and the buffer
outside the slot against the zeros it started from."""
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _example() -> str:
    text = open(os.path.join(ROOT, "README.md")).read()
    start = text.index("```python\n") + len("```python\n")
    return text[start:text.index("```", start)]


def test_readme_example_runs():
    ns = {}
    exec(compile(_example(), "README example", "exec"), ns)
    lay, rank, S = ns["lay"], ns["rank"], ns["S"]
    master, m, v, weights = ns["master"], ns["m"], ns["v"], ns["weights"]
    assert S == 16016 and lay.n_pad == 4 * S
    assert torch.isfinite(master).all() and (v >= 0).all() and (m != 0).any()
    slot = weights[rank * S:(rank + 1) * S]
    assert torch.equal(slot.view(torch.int16), master.to(torch.bfloat16).view(torch.int16))
    outside = torch.cat([weights[:rank * S], weights[(rank + 1) * S:]])
    assert torch.equal(outside.view(torch.int16), torch.zeros_like(outside.view(torch.int16)))
