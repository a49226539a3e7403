"""Synthetic workloads: parameter-list shapes and the input recipe of each
configuration.  Shapes only, no weights: every value is drawn by the seeded
generator.  Nothing here computes the optimizer step or the shard layout.

Parameter lists (registration order; only the segment map depends on it):
  - Llama-shaped 7B: embed [32000 x 4096]; per layer (32) q, k, v, o
    [4096 x 4096], gate, up [11008 x 4096], down [4096 x 11008], input and
    post-attention norms [4096]; final norm [4096]; untied lm_head
    [32000 x 4096]; no biases.  6,738,415,616 parameters.
  - GPT-2-XL-shaped: wte [50257 x 1600], wpe [1024 x 1600]; per layer (48)
    ln_1 w, b, attention c_attn w [1600 x 4800] + b, c_proj w [1600 x 1600]
    + b, ln_2 w, b, mlp c_fc w [1600 x 6400] + b, c_proj w [6400 x 1600] + b;
    ln_f w, b; head tied to wte.  1,557,611,200 parameters.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

from .synth_const import BF16, F16, F32, outlier_threshold


def llama7b_numels() -> List[int]:
    d, ffn, vocab, layers = 4096, 11008, 32000, 32
    out = [vocab * d]
    for _ in range(layers):
        out += [d * d] * 4 + [ffn * d, ffn * d, d * ffn, d, d]
    out += [d, vocab * d]
    return out


def llama7b_shapes() -> List[Tuple[int, int]]:
    """The 7B list as (rows, cols): dim 0 of each tensor, and the product of
    its other dimensions (torch Linear weights are [out, in])."""
    d, ffn, vocab, layers = 4096, 11008, 32000, 32
    out = [(vocab, d)]
    for _ in range(layers):
        out += [(d, d)] * 4 + [(ffn, d), (ffn, d), (d, ffn), (d, 1), (d, 1)]
    out += [(d, 1), (vocab, d)]
    return out


def gpt2xl_shapes() -> List[Tuple[int, int]]:
    """The GPT-2-XL list as (rows, cols) (Conv1D weights are [in, out])."""
    d, ffn, vocab, ctx, layers = 1600, 6400, 50257, 1024, 48
    out = [(vocab, d), (ctx, d)]
    for _ in range(layers):
        out += [(d, 1), (d, 1), (d, 3 * d), (3 * d, 1), (d, d), (d, 1), (d, 1), (d, 1),
                (d, ffn), (ffn, 1), (ffn, d), (d, 1)]
    out += [(d, 1), (d, 1)]
    return out


def gpt2xl_numels() -> List[int]:
    d, ffn, vocab, ctx, layers = 1600, 6400, 50257, 1024, 48
    out = [vocab * d, ctx * d]
    for _ in range(layers):
        out += [d, d, d * 3 * d, 3 * d, d * d, d, d, d, d * ffn, ffn, ffn * d, d]
    out += [d, d]
    return out


@dataclass
class GradDraw:
    kind: int             # BF16, F16 or F32
    sigma: float          # standard deviation of the draw
    scale: float = 1.0    # multiplied into sigma (the fp16 loss scale)
    outlier_p: float = 0.0
    outlier_mul: float = 1.0

    @property
    def thr(self) -> int:
        return outlier_threshold(self.outlier_p)

    @property
    def eff_sigma(self) -> float:
        return self.sigma * self.scale


@dataclass
class Workload:
    cid: int
    name: str
    numels: List[int]
    n_dp: int
    rank: int
    grad: GradDraw
    master_sigma: float = 0.02
    warmup_steps: int = 0        # optimizer steps run before the measured ones
    steps: Tuple[int, ...] = (1,)  # measured step counters t
    micro_batches: int = 1
    loss_scale: float = 1.0
    hp: dict = field(default_factory=lambda: dict(lr=1e-4, beta1=0.9, beta2=0.999,
                                                  eps=1e-8, weight_decay=0.1))
    seed: int = 0
    note: Optional[str] = None
    layout: str = "flat"         # "flat" (one vector) or "dim0" (per-parameter)
    comm: str = "16bit"          # "16bit" rows / weights, or "q8" (8-bit blockwise, ZeRO++)
    controls: bool = False       # global-norm clipping and a dynamic loss scale on the device
    shapes: Optional[List[Tuple[int, int]]] = None


def workloads() -> List[Workload]:
    """The configurations, in order."""
    l7 = llama7b_numels()
    return [
        Workload(0, "tiny_n10000_ndp4", [10000], 4, 1, GradDraw(BF16, 1e-3),
                 steps=(1, 2, 3)),
        Workload(1, "gpt2xl_ndp1", gpt2xl_numels(), 1, 0, GradDraw(BF16, 1e-3),
                 warmup_steps=5, steps=(6,)),
        Workload(2, "llama7b_ndp8_shard", l7, 8, 1,
                 GradDraw(BF16, 1e-3, outlier_p=0.01, outlier_mul=100.0),
                 steps=tuple(range(1, 11))),
        Workload(3, "llama7b_ndp64_shard", l7, 64, 1, GradDraw(BF16, 1e-3),
                 warmup_steps=9, steps=(10,)),
        Workload(4, "llama7b_ndp8_fp16_accum4", l7, 8, 1,
                 GradDraw(F16, 1e-3, scale=65536.0), micro_batches=4,
                 loss_scale=65536.0, steps=(1,)),
        Workload(5, "llama7b_dim0_ndp8_fp32grad", l7, 8, 1,
                 GradDraw(F32, 1e-3, outlier_p=0.01, outlier_mul=100.0), steps=(1, 2, 3),
                 layout="dim0", shapes=llama7b_shapes(),
                 note="per-parameter dim-0 sharding (FSDP2), fp32 gradient rows"),
        Workload(6, "llama7b_ndp8_q8", l7, 8, 1,
                 GradDraw(F32, 1e-3, outlier_p=0.01, outlier_mul=100.0), steps=(1, 2),
                 comm="q8",
                 note="8-bit blockwise rows in, 8-bit weights out (ZeRO++ quantized "
                      "reduce-scatter and all-gather); rows quantized from fp32 draws"),
        Workload(7, "llama7b_ndp8_fp16_accum4_clip", l7, 8, 1,
                 GradDraw(F16, 1e-3, scale=65536.0), micro_batches=4,
                 loss_scale=65536.0, steps=(1,), controls=True,
                 note="configuration 4 with the step controls: the last reduce sums the "
                      "squares, AdamW clips to global norm 1.0 with the device-resident "
                      "dynamic loss scale, and the scale is updated on the device"),
    ]


def workload(cid: int) -> Workload:
    return workloads()[cid]
