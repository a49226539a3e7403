"""The usage example in README.md runs as written (small shapes, three
steps) and does what its comments say: the weights' slot holds the bf16
cast of the updated master, nothing else in the buffer is touched."""
import os
import re

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_runs():
    text = open(os.path.join(ROOT, "README.md"), encoding="utf-8").read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert len(blocks) == 1
    ns = {}
    exec(compile(blocks[0], "README.md", "exec"), ns)
    zs, lay, rank, S = ns["zs"], ns["lay"], ns["rank"], ns["S"]
    master, weights = ns["master"], ns["weights"]
    assert lay.n == 1000 * 64 + 64 and lay.n_dp == 4 and S * 4 == lay.n_pad
    w = weights.float().cpu()
    want = master.to(torch.bfloat16).float().cpu()
    assert torch.equal(w[rank * S:(rank + 1) * S], want)
    assert torch.count_nonzero(w[:rank * S]) == 0 and torch.count_nonzero(w[(rank + 1) * S:]) == 0
    assert int(ns["t"]) == 3 and isinstance(zs.AdamWHParams(step=1), zs.AdamWHParams)
