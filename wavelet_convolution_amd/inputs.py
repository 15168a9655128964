"""Seeded synthetic inputs for the WTConv layer.

This module draws random numbers and converts storage formats. It holds none
of the layer's arithmetic, so both the HIP path and the CPU oracle can be fed
from it without sharing any of the method.

Recipe (one numpy ``default_rng(seed)`` PCG64 stream, drawn in this order):
    x       ~ N(0, 1)          [B, C, H, W]
    dy      ~ N(0, 1)          [B, C, H, W]
    w_base  ~ N(0, 0.02^2)     [C, kb, kb]
    w_lvl   ~ N(0, 0.02^2)     [L, C, 4, k, k]
    scale   ~ U(0.5, 1.5)      [L, C, 4]
Everything is drawn in fp64. Parameters are rounded to fp32. Activations are
rounded to fp32 and then, for bf16 workloads, to bf16 with
round-to-nearest-even; bf16 values are kept as their uint16 bit patterns.
Large tensors are drawn in chunks; numpy fills the stream sequentially, so the
values equal those of one large draw.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

_CHUNK = 1 << 24


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even); return uint16 bits.

    Inputs here are finite, so NaN handling is not needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float, dtype) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=dtype)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        out[lo:hi] = std * rng.standard_normal(hi - lo)
    return out.reshape(shape)


@dataclass
class WTConvInputs:
    """One seeded problem. Activations are fp32 arrays, or uint16 bf16 bits
    when ``dtype == 'bf16'``; parameters are always fp32."""
    B: int
    C: int
    H: int
    W: int
    L: int
    kb: int
    k: int
    dtype: str
    x: np.ndarray
    dy: np.ndarray
    w_base: np.ndarray
    w_lvl: np.ndarray
    scale: np.ndarray

    def act_f64(self, name: str) -> np.ndarray:
        """The activation exactly as the GPU sees it, decoded to fp64."""
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    def params_f64(self):
        return (self.w_base.astype(np.float64), self.w_lvl.astype(np.float64),
                self.scale.astype(np.float64))


def make_inputs(B: int, C: int, H: int, W: int, L: int, kb: int = 5, k: int = 5,
                dtype: str = "f32", seed: int = 0, w_std: float = 0.02,
                scale_lo: float = 0.5, scale_hi: float = 1.5) -> WTConvInputs:
    assert dtype in ("f32", "bf16"), dtype
    rng = np.random.default_rng(seed)
    act_shape = (B, C, H, W)
    x = _normal(rng, act_shape, 1.0, np.float32)
    dy = _normal(rng, act_shape, 1.0, np.float32)
    w_base = (w_std * rng.standard_normal((C, kb, kb))).astype(np.float32)
    w_lvl = (w_std * rng.standard_normal((L, C, 4, k, k))).astype(np.float32)
    scale = rng.uniform(scale_lo, scale_hi, size=(L, C, 4)).astype(np.float32)
    if dtype == "bf16":
        x = f32_to_bf16_bits(x)
        dy = f32_to_bf16_bits(dy)
    return WTConvInputs(B, C, H, W, L, kb, k, dtype, x, dy, w_base, w_lvl, scale)
