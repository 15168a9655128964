"""The WTConv workloads this library is measured and parity-tested on.

Shapes follow the evaluation that the abstract of arXiv:2608.10805 describes
(the WTConvNeXt setting, over several decomposition levels and many tensor
shapes): ConvNeXt stage-like shapes, a level sweep and a large plane. All use x, dy ~ N(0,1), kernels ~ N(0, 0.02^2), scales ~ U(0.5, 1.5),
zero 'same' padding, seed 0.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    B: int
    C: int
    H: int
    W: int
    L: int
    kb: int
    k: int
    dtype: str          # activation storage: "f32" or "bf16"; accumulation is fp32

    @property
    def N(self) -> int:
        return self.B * self.C * self.H * self.W

    def describe(self) -> str:
        return (f"{self.name}: B={self.B} C={self.C} H=W={self.H} L={self.L} "
                f"k_base={self.kb} k_level={self.k} {self.dtype}")


CONFIGS = {
    "tiny_f32": WorkloadConfig("tiny_f32", 1, 8, 32, 32, 2, 5, 5, "f32"),
    "stage1_56": WorkloadConfig("stage1_56", 64, 96, 56, 56, 3, 5, 5, "bf16"),
    "stage2_28": WorkloadConfig("stage2_28", 64, 192, 28, 28, 2, 5, 5, "bf16"),
    "stage3_14": WorkloadConfig("stage3_14", 64, 384, 14, 14, 1, 5, 5, "bf16"),
    **{f"sweep128_L{L}": WorkloadConfig(f"sweep128_L{L}", 32, 128, 128, 128, L, 5, 5, "bf16")
       for L in range(1, 6)},
    "large256": WorkloadConfig("large256", 16, 256, 256, 256, 4, 7, 5, "bf16"),
    # context: the stage-1 activations through the plain depthwise 5x5
    # convolution WTConv stands in for (the layer at L = 0)
    "depthwise56": WorkloadConfig("depthwise56", 64, 96, 56, 56, 0, 5, 5, "bf16"),
}

# the workload the headline images/s figure is quoted on: the largest
# single-GPU configuration (16 x 256 x 256², L4, 7x7 base, 5x5 levels)
HEADLINE = "large256"

# the bar workloads besides the headline (ConvNeXt stage shapes and the level
# sweep), each timed briefly in the same run
BAR_WORKLOADS = ("stage1_56", "stage2_28", "stage3_14", "sweep128_L1", "sweep128_L2", "sweep128_L3",
                 "sweep128_L4", "sweep128_L5")

# the drop-in block timed as context: a ConvNeXt-style block at the stage-1 shape
BLOCK_WORKLOAD = "stage1_56"


def get_config(name: str) -> WorkloadConfig:
    return CONFIGS[name]
