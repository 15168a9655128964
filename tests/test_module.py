"""The drop-in layer (autograd Function + nn.Module over the C-ABI).

CPU: construction, parameter shapes and initialisation, the refusal of CPU
tensors (there is no CPU path), and what a plain autograd composition of the
layer keeps between forward and backward, against the x alone that the
drop-in layer keeps. GPU: forward and every gradient against the oracle, and
the saved tensors and peak memory of one training step."""
import numpy as np
import pytest
import torch

import oracle
from tests._util import TOL, rel_err, to_device, to_f64
from wavelet_convolution_amd.inputs import make_inputs
from wavelet_convolution_amd.module import WTConv2d, WTConvFunction


def test_module_parameters_and_init():
    m = WTConv2d(6, 3, k_base=7, k_level=5)
    assert tuple(m.w_base.shape) == (6, 7, 7)
    assert tuple(m.w_lvl.shape) == (3, 6, 4, 5, 5)
    assert tuple(m.scale.shape) == (3, 6, 4)
    assert all(p.dtype == torch.float32 for p in m.parameters())
    assert float(m.w_base.detach().abs().max()) <= 1 / 7 and float(m.w_lvl.detach().abs().max()) <= 1 / 5
    assert torch.equal(m.scale, torch.ones_like(m.scale))
    # C (k_b^2 + 4 L (k^2 + 1)) parameters: linear in the levels
    assert sum(p.numel() for p in m.parameters()) == 6 * (49 + 4 * 3 * (25 + 1))
    with pytest.raises(ValueError):
        WTConv2d(4, 2, k_base=4)


def test_module_optional_bias_and_base_scale():
    m = WTConv2d(6, 3, k_base=7, k_level=5, bias=True, base_scale=True)
    assert tuple(m.bias.shape) == (6,) and tuple(m.base_scale.shape) == (6,)
    assert torch.equal(m.bias, torch.zeros(6)) and torch.equal(m.base_scale, torch.ones(6))
    assert sum(p.numel() for p in m.parameters()) == 6 * (49 + 4 * 3 * (25 + 1)) + 2 * 6
    plain = WTConv2d(6, 3)
    assert plain.bias is None and plain.base_scale is None


def test_module_refuses_cpu_tensors():
    m = WTConv2d(2, 1)
    with pytest.raises(RuntimeError, match="GPU"):
        m(torch.zeros(1, 2, 8, 8))
    with pytest.raises(ValueError):
        m(torch.zeros(1, 3, 8, 8))


def _saved_bytes(fn, *args):
    """Bytes of the tensors autograd keeps for the backward pass of fn(*args)
    (parameters and inputs excluded: both exist anyway)."""
    keep = {id(a) for a in args}
    total = [0]

    def pack(t):
        if id(t) not in keep and t.data_ptr() not in {a.data_ptr() for a in args}:
            total[0] += t.numel() * t.element_size()
        return t

    with torch.autograd.graph.saved_tensors_hooks(pack, lambda t: t):
        fn(*args)
    return total[0]


def test_plain_composition_keeps_many_activations():
    """A plain autograd composition of the layer (strided grouped conv for
    the analysis, grouped conv per band, transposed conv for the synthesis)
    keeps its bands and intermediate results for the backward pass; the
    drop-in layer keeps x alone. One stage-1 image (96 x 56 x 56, L = 3)."""
    from tests.test_oracle import _torch_layer
    C, H, L = 96, 56, 3
    x = torch.randn(1, C, H, H, dtype=torch.float32, requires_grad=True)
    wb = torch.randn(C, 5, 5, requires_grad=True)
    wl = torch.randn(L, C, 4, 5, 5, requires_grad=True)
    sc = torch.randn(L, C, 4, requires_grad=True)
    kept = _saved_bytes(_torch_layer, x, wb, wl, sc)
    x_bytes = x.numel() * 4
    print(f"plain composition keeps {kept / x_bytes:.2f} x the bytes of x")
    assert kept >= 2 * x_bytes


torch_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")


@pytest.mark.gpu
@torch_gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 3, 32, 32, 2, 5, 5), (2, 3, 56, 56, 3, 5, 5)],
                         ids=lambda s: "x".join(map(str, s)))
def test_module_matches_oracle(shape, dtype):
    B, C, H, W, L, kb, k = shape
    print(f"[module] {dtype} {shape}", flush=True)
    inp = make_inputs(B, C, H, W, L, kb, k, dtype=dtype, seed=20)
    x, dy, wb, wl, sc = to_device(inp)
    m = WTConv2d(C, L, kb, k, device="cuda")
    with torch.no_grad():
        m.w_base.copy_(wb)
        m.w_lvl.copy_(wl)
        m.scale.copy_(sc)
    x.requires_grad_(True)
    y = m(x)
    y.backward(dy)
    torch.cuda.synchronize()
    xo, dyo = inp.act_f64("x"), inp.act_f64("dy")
    wbo, wlo, sco = inp.params_f64()
    tol = TOL[dtype]
    assert y.dtype == x.dtype and x.grad.dtype == x.dtype
    assert rel_err(to_f64(y), oracle.fwd(xo, wbo, wlo, sco)) <= tol
    assert rel_err(to_f64(x.grad), oracle.bwd_data(dyo, wbo, wlo, sco)) <= tol
    gb, gl, gs = oracle.bwd_weight(xo, dyo, wbo, wlo, sco)
    assert rel_err(to_f64(m.w_base.grad), gb) <= TOL["f32"]
    assert rel_err(to_f64(m.w_lvl.grad), gl) <= TOL["f32"]
    assert rel_err(to_f64(m.scale.grad), gs) <= TOL["f32"]


@pytest.mark.gpu
@torch_gpu
def test_module_bias_and_base_scale_match_oracle():
    """With the optional bias and base scale: y = layer(x; w_base * s_b) + b,
    and the gradients of b (the sum of dy per channel), of s_b
    (sum(dw_base_eff * w_base) per channel) and of w_base (dw_base_eff * s_b),
    all from the oracle's gradients."""
    B, C, H, W, L, kb, k = 2, 3, 32, 32, 2, 5, 5
    inp = make_inputs(B, C, H, W, L, kb, k, dtype="f32", seed=21)
    x, dy, wb, wl, sc = to_device(inp)
    m = WTConv2d(C, L, kb, k, device="cuda", bias=True, base_scale=True)
    rng = np.random.default_rng(5)
    bias = rng.standard_normal(C)
    bscale = rng.uniform(0.5, 1.5, C)
    with torch.no_grad():
        m.w_base.copy_(wb)
        m.w_lvl.copy_(wl)
        m.scale.copy_(sc)
        m.bias.copy_(torch.from_numpy(bias))
        m.base_scale.copy_(torch.from_numpy(bscale))
    x.requires_grad_(True)
    y = m(x)
    y.backward(dy)
    torch.cuda.synchronize()
    xo, dyo = inp.act_f64("x"), inp.act_f64("dy")
    wbo, wlo, sco = inp.params_f64()
    wbe = wbo * bscale[:, None, None]
    yo = oracle.fwd(xo, wbe, wlo, sco) + bias[None, :, None, None]
    assert rel_err(to_f64(y), yo) <= TOL["f32"]
    assert rel_err(to_f64(x.grad), oracle.bwd_data(dyo, wbe, wlo, sco)) <= TOL["f32"]
    gbe, gl, gs = oracle.bwd_weight(xo, dyo, wbe, wlo, sco)
    assert rel_err(to_f64(m.bias.grad), dyo.sum(axis=(0, 2, 3))) <= TOL["f32"]
    assert rel_err(to_f64(m.base_scale.grad), (gbe * wbo).sum(axis=(1, 2))) <= TOL["f32"]
    assert rel_err(to_f64(m.w_base.grad), gbe * bscale[:, None, None]) <= TOL["f32"]
    assert rel_err(to_f64(m.w_lvl.grad), gl) <= TOL["f32"]
    assert rel_err(to_f64(m.scale.grad), gs) <= TOL["f32"]


@pytest.mark.gpu
@torch_gpu
def test_module_channels_last():
    """A channels-last input gives the same results as the planar one, and y
    and dx keep its memory order."""
    print("[module] channels last 2x3x28x28 L2 f32", flush=True)
    inp = make_inputs(2, 3, 28, 28, 2, 5, 5, dtype="f32", seed=21)
    x, dy, wb, wl, sc = to_device(inp)
    m = WTConv2d(3, 2, 5, 5, device="cuda")
    outs = []
    for fmt in (torch.contiguous_format, torch.channels_last):
        xi = x.detach().contiguous(memory_format=fmt).requires_grad_(True)
        m.zero_grad()
        y = m(xi)
        y.backward(dy.contiguous(memory_format=fmt))
        torch.cuda.synchronize()
        assert y.is_contiguous(memory_format=fmt) and xi.grad.is_contiguous(memory_format=fmt)
        outs.append([to_f64(t) for t in (y, xi.grad, m.w_base.grad, m.w_lvl.grad, m.scale.grad)])
    for a, b in zip(*outs):
        assert rel_err(b, a) <= 1e-5


@pytest.mark.gpu
@torch_gpu
def test_module_keeps_only_x_and_its_peak_memory():
    """The backward pass rebuilds the pyramid on chip: autograd holds x (and
    the parameters), nothing else. Peak memory of a training step stays
    within x, y, dy, dx, the gradients and the workspace."""
    print("[module] saved tensors and peak memory, 16x96x56x56 L3 bf16", flush=True)
    B, C, H, L = 16, 96, 56, 3
    m = WTConv2d(C, L, device="cuda")
    x = torch.randn(B, C, H, H, device="cuda").to(torch.bfloat16).requires_grad_(True)
    params = {p.data_ptr() for p in m.parameters()}
    saved = []

    def pack(t):
        saved.append(t)
        return t

    with torch.autograd.graph.saved_tensors_hooks(pack, lambda t: t):
        y = m(x)
    extra = [t for t in saved if t.data_ptr() != x.data_ptr() and t.data_ptr() not in params]
    assert not extra, [tuple(t.shape) for t in extra]
    dy = torch.randn_like(y)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    y.backward(dy)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    act = x.numel() * x.element_size()
    print(f"backward peak above the live tensors: {peak / act:.2f} x the bytes of x", flush=True)
    # dx, the three gradients, the weight-gradient workspace and allocator rounding
    assert peak <= 2.5 * act + 16 * 2 ** 20


@pytest.mark.gpu
@torch_gpu
def test_module_trains():
    """A few plain SGD steps fitting the layer to a target made by another
    instance of it: the loss falls steadily (autograd wiring, gradient
    accumulation into .grad, parameter updates between calls)."""
    print("[module] training 4x8x28x28 L2 f32", flush=True)
    torch.manual_seed(0)
    teacher = WTConv2d(8, 2, 5, 5, device="cuda")
    student = WTConv2d(8, 2, 5, 5, device="cuda")
    x = torch.randn(4, 8, 28, 28, device="cuda")
    with torch.no_grad():
        target = teacher(x)
    opt = torch.optim.SGD(student.parameters(), lr=0.5)
    losses = []
    for _ in range(30):
        opt.zero_grad()
        loss = torch.nn.functional.mse_loss(student(x), target)
        loss.backward()
        opt.step()
        losses.append(float(loss.detach()))
    print(f"loss {losses[0]:.4g} -> {losses[-1]:.4g}", flush=True)
    assert losses[-1] < 0.25 * losses[0]
    assert all(b <= a * 1.0001 for a, b in zip(losses, losses[1:]))
