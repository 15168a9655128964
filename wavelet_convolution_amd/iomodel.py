"""Analytic I/O and arithmetic model of one WTConv training step.

The abstract of arXiv:2608.10805 models WTConv's I/O to locate its HBM
bottleneck; this is this library's own model of the same kind, for
the three-call step (forward, backward data, backward weight).

Minimum HBM bytes: what the method must move if every intermediate stays on
chip. Forward reads x and writes y; backward data reads dy and writes dx;
backward weight reads x and dy and writes the gradients. Parameters are
read by each call.

Arithmetic: each call does (kb^2 + k^2 * S_L) multiply-adds per activation
element, S_L = sum_{l=1..L} 4^(1-l): level l convolves 4 bands of N / 4^l
positions with k x k kernels. The Haar butterflies add about one add per
subband coefficient and are not counted.

Naive model: one kernel per step with every intermediate in HBM (fp32
intermediates), as the naive chain in this library does.
"""
from __future__ import annotations

from dataclasses import dataclass

HBM_PEAK_TBS = 8.0            # MI355X HBM3E, TB/s
FP32_VECTOR_PEAK_TFLOPS = 157.3   # MI355X published fp32 vector peak (packed FMA)
FP32_UNPACKED_FMA_TFLOPS = 78.6   # 256 CU x 64 lanes x 2 flop x 2.4 GHz (one FMA per lane-cycle)


def s_levels(L: int) -> float:
    return sum(4.0 ** (1 - l) for l in range(1, L + 1))


@dataclass(frozen=True)
class StepModel:
    N: int
    elem_bytes: int
    param_bytes: int
    mac_per_call: float

    @property
    def flops_per_call(self) -> float:
        return 2.0 * self.mac_per_call

    @property
    def fwd_bytes(self) -> int:
        return 2 * self.N * self.elem_bytes + self.param_bytes

    @property
    def bwd_data_bytes(self) -> int:
        return 2 * self.N * self.elem_bytes + self.param_bytes

    @property
    def bwd_weight_bytes(self) -> int:
        return 2 * self.N * self.elem_bytes + 2 * self.param_bytes

    @property
    def step_bytes(self) -> int:
        return self.fwd_bytes + self.bwd_data_bytes + self.bwd_weight_bytes

    @property
    def bwd_fused_bytes(self) -> int:
        """One backward call for dx and every weight gradient: x and dy read
        once, dx written once, the parameters read, the gradients written."""
        return 3 * self.N * self.elem_bytes + 2 * self.param_bytes

    @property
    def step_bytes_fused_bwd(self) -> int:
        """Forward plus the single-call backward: 5 N e + 3 P."""
        return self.fwd_bytes + self.bwd_fused_bytes

    @property
    def step_flops(self) -> float:
        return 3.0 * self.flops_per_call


def param_count(C: int, L: int, kb: int, k: int) -> int:
    return C * (kb * kb + 4 * L * (k * k + 1))


def step_model(B: int, C: int, H: int, W: int, L: int, kb: int, k: int, dtype: str) -> StepModel:
    N = B * C * H * W
    e = 2 if dtype == "bf16" else 4
    macs = (kb * kb + k * k * s_levels(L)) * N
    return StepModel(N=N, elem_bytes=e, param_bytes=4 * param_count(C, L, kb, k), mac_per_call=macs)


def naive_fwd_bytes(B: int, C: int, H: int, W: int, L: int, dtype: str) -> int:
    """Bytes the one-kernel-per-step chain moves in a forward pass.

    Per level l (N_l = N / 4^(l-1) values at the level's input resolution):
    analysis reads N_l and writes N_l, the convolution reads and writes N_l,
    the scale reads and writes N_l, the LL add reads 2 N_l / 4 and writes
    N_l / 4 (all but the coarsest level), synthesis reads and writes N_l.
    Then the base convolution reads x and writes N, and the final add reads
    2N and writes y. Intermediates are fp32, activations dtype."""
    N = B * C * H * W
    e = 2 if dtype == "bf16" else 4
    f = 4
    total = 0.0
    for l in range(1, L + 1):
        Nl = N / 4 ** (l - 1)
        src = e if l == 1 else f
        total += Nl * src + Nl * f          # analysis
        total += 2 * Nl * f                 # convolution
        total += 2 * Nl * f                 # scale
        if l < L:
            total += 3 * (Nl / 4) * f       # LL add
        total += 2 * Nl * f                 # synthesis
    total += N * e + N * f                  # base convolution
    total += 2 * N * f + N * e              # final add
    return int(total)
