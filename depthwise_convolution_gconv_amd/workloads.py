"""Seeded synthetic workloads for grouped-convolution forward.

This module only draws and quantises inputs; it holds none of the convolution's
arithmetic.  Both the HIP path's tests and the oracle's tests take their inputs
from here, so the two sides see bit-identical operands.

Recipe (the same for every workload):

* ``numpy.random.default_rng(seed).standard_normal(shape, dtype=float32)``,
  scaled by the standard deviation ``sqrt(var)`` (the variance notation N(0, v)
  is read as variance: 1/36, 1/1152, 1/31 and 1/288 are each 1/(C/g*KH*KW), the
  fan-in, which keeps outputs near unit variance);
* cast to the storage dtype with round-to-nearest-even (``torch.Tensor.to`` on
  the CPU);
* seeds: x = 1000 + i, w = 2000 + i, bias = 3000 + i for workload number i.

The shapes are those of the pages' workloads: the layer timed in the
discuss.pytorch.org thread "F.conv2d runs x15 slower in mixed-precision/
half-precision mode" (x [1,512,256,256], w [512,128,3,3], groups=4, padding 3//2),
a Conformer depthwise conv over (batch, steps, channels) from speechbrain issue
#2733, a fully grouped ResNeXt-style layer (neon issue "Grouped convolutions"),
and a model ensemble folded into groups (functorch issue #365, the conv batching
rule).  No dataset is involved; all values are synthetic.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int                    # seed offset
    layout: str                   # "nchw", "nhwc" or "ntc"
    x_shape: Tuple[int, ...]
    w_shape: Tuple[int, ...]
    groups: int
    stride: int
    pad: int
    dilation: int
    dtype: str                    # "f32" | "f16" | "bf16"
    var_x: float
    var_w: float
    var_b: Optional[float]        # None: no bias
    what: str = ""

    @property
    def has_bias(self) -> bool:
        return self.var_b is not None

    @property
    def bias_shape(self) -> Tuple[int, ...]:
        return (self.w_shape[0],)


WORKLOADS = {
    "c1_g4_f32": Workload(
        "c1_g4_f32", 1, "nchw", (1, 16, 32, 32), (16, 4, 3, 3), 4, 1, 1, 1, "f32",
        1.0, 1 / 36, None, "small grouped conv2d, g=4"),
    "c2_p2layer_f32": Workload(
        "c2_p2layer_f32", 2, "nchw", (1, 512, 256, 256), (512, 128, 3, 3), 4, 1, 1, 1, "f32",
        1.0, 1 / 1152, None, "the discuss.pytorch.org layer, fp32"),
    "c2_p2layer_f16": Workload(
        "c2_p2layer_f16", 2, "nchw", (1, 512, 256, 256), (512, 128, 3, 3), 4, 1, 1, 1, "f16",
        1.0, 1 / 1152, None, "the discuss.pytorch.org layer, fp16 in / fp32 accumulate"),
    "c3_dw1d_btc_f32": Workload(
        "c3_dw1d_btc_f32", 3, "ntc", (8, 1024, 512), (512, 1, 31), 512, 1, 15, 1, "f32",
        1.0, 1 / 31, 0.01, "Conformer depthwise conv1d, (batch, steps, channels)"),
    "c4_fullgroup_bf16": Workload(
        "c4_fullgroup_bf16", 4, "nchw", (32, 1024, 14, 14), (1024, 4, 3, 3), 256, 1, 1, 1, "bf16",
        1.0, 1 / 36, 0.01, "fully grouped conv2d, 4 in / 4 out channels per group"),
    "c5_ensemble_f16": Workload(
        "c5_ensemble_f16", 5, "nchw", (64, 1024, 28, 28), (2048, 32, 3, 3), 32, 1, 1, 1, "f16",
        1.0, 1 / 288, 0.01, "32-model ensemble folded into groups"),
}

HEADLINE = "c2_p2layer_f16"

# Strided depthwise layers (the depthwise-separable downsampling that speechbrain
# issue #2733 names as the next candidate: Fast Conformer's subsampling CNN, which
# needs stride).  Shapes of a Fast Conformer subsampling stage on 8 utterances:
# 256 channels, 512 frames x 40 frequency bins in, a 3x3 depthwise filter with
# stride 2 and padding 1; the stride-1 layer on the same input; and the
# Conformer's 1-D depthwise conv with stride 2.
NEXT_WORKLOADS = {
    "n1_dw2d_s2_f32": Workload(
        "n1_dw2d_s2_f32", 11, "nchw", (8, 256, 512, 40), (256, 1, 3, 3), 256, 2, 1, 1, "f32",
        1.0, 1 / 9, 0.01, "depthwise 3x3 conv2d, stride 2 (subsampling stage)"),
    "n2_dw2d_s2_bf16": Workload(
        "n2_dw2d_s2_bf16", 12, "nchw", (8, 256, 512, 40), (256, 1, 3, 3), 256, 2, 1, 1, "bf16",
        1.0, 1 / 9, 0.01, "depthwise 3x3 conv2d, stride 2, bf16"),
    "n3_dw2d_s1_f32": Workload(
        "n3_dw2d_s1_f32", 13, "nchw", (8, 256, 512, 40), (256, 1, 3, 3), 256, 1, 1, 1, "f32",
        1.0, 1 / 9, 0.01, "depthwise 3x3 conv2d, stride 1"),
    # The same stage in the channels-last (NHWC) layout: x [8, 512, 40, 256],
    # w [256, 3, 3, 1].
    "n7_dw2d_nhwc_s2_f32": Workload(
        "n7_dw2d_nhwc_s2_f32", 17, "nhwc", (8, 512, 40, 256), (256, 3, 3, 1), 256, 2, 1, 1, "f32",
        1.0, 1 / 9, 0.01, "depthwise 3x3 conv2d over channels-last tensors, stride 2"),
    "n8_dw2d_nhwc_s1_bf16": Workload(
        "n8_dw2d_nhwc_s1_bf16", 18, "nhwc", (8, 512, 40, 256), (256, 3, 3, 1), 256, 1, 1, 1, "bf16",
        1.0, 1 / 9, 0.01, "depthwise 3x3 conv2d over channels-last tensors, stride 1, bf16"),
    # The 32-model ensemble layer in the channels-last layout: x [64, 28, 28, 1024],
    # w [2048, 3, 3, 32], groups 32.
    "n9_ensemble_nhwc_f16": Workload(
        "n9_ensemble_nhwc_f16", 19, "nhwc", (64, 28, 28, 1024), (2048, 3, 3, 32), 32, 1, 1, 1, "f16",
        1.0, 1 / 288, 0.01, "32-model ensemble folded into groups, channels-last"),
    # The fully grouped layer (4 in / 4 out per group) in the channels-last layout.
    "n10_fullgroup_nhwc_bf16": Workload(
        "n10_fullgroup_nhwc_bf16", 20, "nhwc", (32, 14, 14, 1024), (1024, 3, 3, 4), 256, 1, 1, 1, "bf16",
        1.0, 1 / 36, 0.01, "fully grouped conv2d, 4 in / 4 out per group, channels-last"),
    "n4_dw1d_s2_f32": Workload(
        "n4_dw1d_s2_f32", 14, "ntc", (8, 1024, 512), (512, 1, 31), 512, 2, 15, 1, "f32",
        1.0, 1 / 31, 0.01, "depthwise conv1d, (batch, steps, channels), stride 2"),
}


def draw(shape, var: float, seed: int, dtype: str) -> torch.Tensor:
    """Seeded N(0, var) draw in fp32, rounded to `dtype` (RNE), as a CPU tensor."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(tuple(shape), dtype=np.float32)
    a *= np.float32(math.sqrt(var))
    return torch.from_numpy(a).to(DTYPES[dtype])


def make_inputs(wl: Workload, seed_shift: int = 0):
    """(x, w, bias-or-None) as CPU tensors of the workload's dtype."""
    x = draw(wl.x_shape, wl.var_x, 1000 + wl.index + seed_shift, wl.dtype)
    w = draw(wl.w_shape, wl.var_w, 2000 + wl.index + seed_shift, wl.dtype)
    b = draw(wl.bias_shape, wl.var_b, 3000 + wl.index + seed_shift, wl.dtype) if wl.has_bias else None
    return x, w, b


def as_f64(t: Optional[torch.Tensor]):
    """Exact widening of a CPU tensor to a float64 numpy array (None passes)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
