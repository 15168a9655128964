"""Drop-in WTConv layer for PyTorch: an autograd Function and an nn.Module
over the C-ABI entry points.

The forward pass keeps only x (and the parameters) for the backward pass:
``wtconv_bwd_data`` and ``wtconv_bwd_weight`` rebuild the Haar pyramid of x
and dy on chip, so no band tensor is stored between the passes. Every step
of the computation runs in libwtconv.so; this file allocates outputs and
marshals arguments only. Tensors must be on the GPU: there is no CPU path.

Layer (abstract of arXiv:2608.10805, the tech.sinsc.com page): a depthwise
k_base x k_base convolution plus an L-level Haar branch, each level's four
subbands convolved depthwise (k_level x k_level) and scaled per channel and
band, the results synthesised back in one closed-form pass.
"""
from __future__ import annotations

import math

import torch

from . import binding as _b


def _check_device(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise RuntimeError("WTConv runs on the GPU only (libwtconv.so); got a tensor on "
                               f"{t.device} - there is no CPU implementation")


def _order(x: torch.Tensor):
    """channels_last if x is stored that way (and not also planar), else planar."""
    if not x.is_contiguous() and x.dim() == 4 and x.is_contiguous(memory_format=torch.channels_last):
        return torch.channels_last
    return torch.contiguous_format


class WTConvFunction(torch.autograd.Function):
    """y = WTConv(x; w_base, w_lvl, scale).

    x: [B, C, H, W] fp32 or bf16, w_base: [C, kb, kb], w_lvl:
    [L, C, 4, k, k], scale: [L, C, 4], all fp32. Gradients of the
    parameters are fp32; the gradient of x has x's dtype. A channels-last x
    keeps its memory order (y and dx are channels last too); the library runs
    the planar kernels on converted copies of it.
    """

    @staticmethod
    def forward(ctx, x, w_base, w_lvl, scale):
        _check_device(x, w_base, w_lvl, scale)
        x = x.contiguous(memory_format=_order(x))
        y = _b.wtconv_fwd(x, w_base, w_lvl, scale)
        ctx.save_for_backward(x, w_base, w_lvl, scale)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, w_base, w_lvl, scale = ctx.saved_tensors
        dy = dy.to(x.dtype).contiguous(memory_format=_order(x))
        dx = dwb = dwl = dsc = None
        if ctx.needs_input_grad[0] and any(ctx.needs_input_grad[1:]):
            # both results: one call (a single pass over x and dy where the library has one)
            dx, (dwb, dwl, dsc) = _b.wtconv_bwd(x, dy, w_base, w_lvl, scale)
        elif ctx.needs_input_grad[0]:
            dx = _b.wtconv_bwd_data(dy, w_base, w_lvl, scale)
        elif any(ctx.needs_input_grad[1:]):
            dwb, dwl, dsc = _b.wtconv_bwd_weight(x, dy, int(w_base.shape[-1]), w_lvl, scale)
        return dx, dwb, dwl, dsc


def wtconv(x, w_base, w_lvl, scale):
    """Functional form of the layer (differentiable)."""
    return WTConvFunction.apply(x, w_base, w_lvl, scale)


class WTConv2d(torch.nn.Module):
    """Depthwise WTConv with `channels` channels and `levels` Haar levels.

    Parameters (fp32): ``w_base`` [C, k_base, k_base], ``w_lvl``
    [L, C, 4, k_level, k_level], ``scale`` [L, C, 4]. Initialisation: both
    kernels like a depthwise ``nn.Conv2d`` (uniform, bound 1/sqrt(k*k)), and
    unit scales. The pages fix no initialisation; this is the plainest one.
    Input and output: [B, C, H, W], fp32 or bf16, any H, W >= 1 ('same'
    zero padding, stride 1; an odd band grid is analysed with one extra zero
    row or column and its synthesis is cropped back).

    Optional extras of a drop-in convolution layer, both off by default (the
    layer the pages describe has neither): ``bias=True`` adds a learned
    per-channel bias ``bias`` [C] to the output, ``base_scale=True`` a learned
    per-channel factor ``base_scale`` [C] on the base convolution's result
    (initialised to 1). The factor is applied by scaling the base kernel
    before the call (``w_base * base_scale``, exact in the result up to fp32
    rounding since the base convolution is linear in its kernel); the bias is
    added to the library's output. Their gradients follow by autograd from
    the library's ``dw_base`` and from the output gradient.
    """

    def __init__(self, channels: int, levels: int, k_base: int = 5, k_level: int = 5,
                 device=None, bias: bool = False, base_scale: bool = False):
        super().__init__()
        if channels < 1 or levels < 0 or k_base % 2 == 0 or k_level % 2 == 0:
            raise ValueError("channels >= 1, levels >= 0 and odd kernel sizes are required")
        self.channels, self.levels, self.k_base, self.k_level = channels, levels, k_base, k_level
        f32 = dict(dtype=torch.float32, device=device)
        self.w_base = torch.nn.Parameter(torch.empty(channels, k_base, k_base, **f32))
        self.w_lvl = torch.nn.Parameter(torch.empty(levels, channels, 4, k_level, k_level, **f32))
        self.scale = torch.nn.Parameter(torch.ones(levels, channels, 4, **f32))
        self.bias = torch.nn.Parameter(torch.zeros(channels, **f32)) if bias else None
        self.base_scale = torch.nn.Parameter(torch.ones(channels, **f32)) if base_scale else None
        self.reset_parameters()

    def reset_parameters(self) -> None:
        with torch.no_grad():
            self.w_base.uniform_(-1.0 / math.sqrt(self.k_base ** 2), 1.0 / math.sqrt(self.k_base ** 2))
            self.w_lvl.uniform_(-1.0 / math.sqrt(self.k_level ** 2), 1.0 / math.sqrt(self.k_level ** 2))
            self.scale.fill_(1.0)
            if self.bias is not None:
                self.bias.zero_()
            if self.base_scale is not None:
                self.base_scale.fill_(1.0)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.dim() != 4 or x.shape[1] != self.channels:
            raise ValueError(f"expected [B, {self.channels}, H, W], got {tuple(x.shape)}")
        w_base = self.w_base
        if self.base_scale is not None:
            w_base = w_base * self.base_scale.view(-1, 1, 1)
        y = WTConvFunction.apply(x, w_base, self.w_lvl, self.scale)
        if self.bias is not None:
            y = y + self.bias.view(1, -1, 1, 1).to(y.dtype)
        return y

    def extra_repr(self) -> str:
        return (f"channels={self.channels}, levels={self.levels}, k_base={self.k_base}, "
                f"k_level={self.k_level}, bias={self.bias is not None}, "
                f"base_scale={self.base_scale is not None}")
