"""GPU parity: the HIP path (through the C-ABI) against the fp64 oracle on
the same seeded inputs.

Bar (normwise max relative error per output tensor, max|g-o| / max|o|):
1e-4 for fp32 activations, 2e-2 for bf16 activations. Every shape is also
run with fp32 activations, where the kernels are the same templates, so a
mistake small enough to hide under the bf16 bound still fails at 1e-4.
"""
import sys

import numpy as np
import pytest

import oracle
from tests._util import TOL, rel_err, to_device, to_f64
from wavelet_convolution_amd.inputs import make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU machines too
    pytest.skip("no GPU", allow_module_level=True)

from wavelet_convolution_amd import binding as wt  # noqa: E402


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# (B, C, H, W, L, kb, k): every whole-plane plan, including shapes with a
# partial last round of work items, other kernel sizes and non-square planes
SMALL = [
    (2, 3, 32, 32, 2, 5, 5),
    (2, 3, 56, 56, 3, 5, 5),
    (2, 3, 28, 28, 2, 5, 5),
    (2, 3, 14, 14, 1, 5, 5),
    (1, 2, 128, 128, 1, 5, 5),
    (1, 2, 128, 128, 3, 5, 5),
    (1, 2, 128, 128, 5, 5, 5),
    (2, 3, 32, 32, 3, 7, 5),
    (2, 3, 24, 40, 3, 3, 3),
    (3, 2, 16, 16, 4, 3, 7),
    (2, 2, 64, 64, 4, 7, 5),
    # planes that take the split path (coarse pass on the level-L0 LL sums,
    # then full-width fine tiles with a halo)
    (2, 3, 64, 64, 4, 3, 3),
    (2, 3, 64, 64, 2, 5, 5),
    # the large-plane column tiles (7x7 base, coarse pass on the level-2 sums;
    # bf16: the matrix-core fine pass and weight gradient), and a batch whose
    # tiles split into several weight-gradient chunks per channel, the last
    # one partial
    (1, 2, 256, 256, 4, 7, 5),
    (3, 5, 256, 256, 4, 7, 5),
    # batches that leave the last multi-plane step of a weight-gradient chunk
    # partly empty (the whole-plane plans take several planes per step)
    (11, 2, 14, 14, 1, 5, 5),
    (7, 3, 28, 28, 2, 5, 5),
    (5, 2, 56, 56, 3, 5, 5),
]



def _oracle_all(inp):
    x, dy = inp.act_f64("x"), inp.act_f64("dy")
    wb, wl, sc = inp.params_f64()
    return (oracle.fwd(x, wb, wl, sc), oracle.bwd_data(dy, wb, wl, sc), oracle.bwd_weight(x, dy, wb, wl, sc))


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_matches_oracle(shape, dtype):
    B, C, H, W, L, kb, k = shape
    _say(f"[parity] fused {dtype} {shape}")
    inp = make_inputs(B, C, H, W, L, kb, k, dtype=dtype, seed=0)
    x, dy, wb, wl, sc = to_device(inp)
    y = wt.wtconv_fwd(x, wb, wl, sc)
    dx = wt.wtconv_bwd_data(dy, wb, wl, sc)
    torch.cuda.synchronize()
    oy, odx, (odwb, odwl, odsc) = _oracle_all(inp)
    tol = TOL[dtype]
    assert rel_err(to_f64(y), oy) <= tol
    assert rel_err(to_f64(dx), odx) <= tol
    dwb, dwl, dsc = wt.wtconv_bwd_weight(x, dy, kb, wl, sc)
    torch.cuda.synchronize()
    # gradients are fp32 sums over the batch of bf16-exact products
    assert rel_err(to_f64(dwb), odwb) <= TOL["f32"]
    assert rel_err(to_f64(dwl), odwl) <= TOL["f32"]
    assert rel_err(to_f64(dsc), odsc) <= TOL["f32"]


@pytest.mark.parametrize("shape", SMALL[:4] + SMALL[7:9], ids=lambda s: "x".join(map(str, s)))
def test_naive_matches_oracle(shape):
    B, C, H, W, L, kb, k = shape
    _say(f"[parity] naive f32 {shape}")
    inp = make_inputs(B, C, H, W, L, kb, k, dtype="f32", seed=1)
    x, dy, wb, wl, sc = to_device(inp)
    y = wt.wtconv_naive_fwd(x, wb, wl, sc)
    dx = wt.wtconv_naive_bwd_data(dy, wb, wl, sc)
    dwb, dwl, dsc = wt.wtconv_naive_bwd_weight(x, dy, kb, wl, sc)
    torch.cuda.synchronize()
    oy, odx, (odwb, odwl, odsc) = _oracle_all(inp)
    for g, o in ((y, oy), (dx, odx), (dwb, odwb), (dwl, odwl), (dsc, odsc)):
        assert rel_err(to_f64(g), o) <= TOL["f32"]


def test_adjoint_identity_on_gpu():
    _say("[parity] adjoint 2x3x56x56 L3")
    inp = make_inputs(2, 3, 56, 56, 3, dtype="f32", seed=2)
    x, dy, wb, wl, sc = to_device(inp)
    y = wt.wtconv_fwd(x, wb, wl, sc)
    dx = wt.wtconv_bwd_data(dy, wb, wl, sc)
    lhs = float((y.double() * dy.double()).sum())
    rhs = float((x.double() * dx.double()).sum())
    assert abs(lhs - rhs) <= 1e-5 * (abs(lhs) + abs(rhs) + 1.0)


def test_bwd_weight_bitwise_deterministic():
    _say("[parity] determinism 8x16x56x56 L3 bf16")
    inp = make_inputs(8, 16, 56, 56, 3, dtype="bf16", seed=3)
    x, dy, wb, wl, sc = to_device(inp)
    a = wt.wtconv_bwd_weight(x, dy, 5, wl, sc)
    b = wt.wtconv_bwd_weight(x, dy, 5, wl, sc)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_zero_branch_equals_base_only():
    """Zero scales: the branch contributes exactly nothing (not approximately)."""
    _say("[parity] zero branch")
    inp = make_inputs(2, 3, 56, 56, 3, dtype="f32", seed=4)
    x, dy, wb, wl, sc = to_device(inp)
    y0 = wt.wtconv_fwd(x, wb, wl, torch.zeros_like(sc))
    ref = torch.nn.functional.conv2d(x.double().cpu(), wb.double().cpu()[:, None], padding=2, groups=3)
    assert rel_err(to_f64(y0), ref.numpy()) <= 1e-6


def test_bf16_store_rounding_is_round_to_nearest_even():
    """Pin the fp32 -> bf16 narrowing of the stores bit-exactly: with zero
    scales and a base kernel c * delta, y = c * x is exact in fp32 (8-bit
    times 8-bit significands), so the store's rounding is the only one.
    Expected bits: numpy round-to-nearest-even of the exact product."""
    from wavelet_convolution_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits
    _say("[parity] bf16 RNE store")
    inp = make_inputs(2, 3, 56, 56, 3, dtype="bf16", seed=5)
    x, dy, wb, wl, sc = to_device(inp)
    c = 1.0 + 2.0 ** -8 + 2.0 ** -7   # many products land exactly on bf16 ties
    wdelta = torch.zeros_like(wb)
    wdelta[:, 2, 2] = c
    y = wt.wtconv_fwd(x, wdelta, wl, torch.zeros_like(sc))
    torch.cuda.synchronize()
    exact = bf16_bits_to_f32(inp.x).astype(np.float64) * c
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)   # exact in fp32
    expect = f32_to_bf16_bits(exact.astype(np.float32))
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("shape", [(2, 3, 56, 56, 3), (1, 2, 128, 128, 5), (1, 2, 64, 64, 4)],
                         ids=lambda s: "x".join(map(str, s)))
def test_identity_levels_closed_form_on_gpu(shape):
    """No oracle involved: with zero base taps, centre-delta level taps and
    unit scales every level reproduces its input, so the layer returns
    sum_{m<L} BlockMean_{2^m}(x) (derived by hand from the cascade). Covers the
    whole-plane and the split path (64x64, L=4, 3x3 taps)."""
    B, C, H, W, L = shape
    k = 3 if H == 64 else 5
    _say(f"[parity] identity levels {shape}")
    inp = make_inputs(B, C, H, W, L, 5 if H != 64 else 3, k, dtype="f32", seed=6)
    x, dy, wb, wl, sc = to_device(inp)
    wl = torch.zeros_like(wl)
    wl[..., k // 2, k // 2] = 1.0
    y = wt.wtconv_fwd(x, torch.zeros_like(wb), wl, torch.ones_like(sc))
    torch.cuda.synchronize()
    xn = inp.x.astype(np.float64)
    expect = np.zeros_like(xn)
    for m in range(L):
        s = 1 << m
        bm = xn.reshape(B, C, H // s, s, W // s, s).mean(axis=(3, 5))
        expect += np.repeat(np.repeat(bm, s, axis=2), s, axis=3)
    assert rel_err(to_f64(y), expect) <= 1e-6


def test_level_zero_and_unplanned_shapes():
    """L = 0 is the plain depthwise convolution. Plane sizes without a fused
    kernel (here 20 x 12 and 24 x 20) run the generic chain through the same
    entry points."""
    _say("[parity] L = 0 and unplanned shapes")
    inp = make_inputs(2, 3, 20, 12, 0, 5, 5, dtype="f32", seed=7)
    x, dy, wb, wl, sc = to_device(inp)
    ref = torch.nn.functional.conv2d(x.double().cpu(), wb.double().cpu()[:, None], padding=2, groups=3)
    for fn in (wt.wtconv_naive_fwd, wt.wtconv_fwd):
        y = fn(x, wb, wl, sc)
        torch.cuda.synchronize()
        assert rel_err(to_f64(y), ref.numpy()) <= 1e-6
    _check_all_three(2, 3, 24, 20, 2, 3, 5)


def _check_all_three(B, C, H, W, L, kb, k, seed=7):
    for dtype in ("f32", "bf16"):
        inp = make_inputs(B, C, H, W, L, kb, k, dtype=dtype, seed=seed)
        x, dy, wb, wl, sc = to_device(inp)
        y = wt.wtconv_fwd(x, wb, wl, sc)
        dx = wt.wtconv_bwd_data(dy, wb, wl, sc)
        dwb, dwl, dsc = wt.wtconv_bwd_weight(x, dy, kb, wl, sc)
        torch.cuda.synchronize()
        oy, odx, (odwb, odwl, odsc) = _oracle_all(inp)
        assert rel_err(to_f64(y), oy) <= TOL[dtype] and rel_err(to_f64(dx), odx) <= TOL[dtype]
        for g, o in ((dwb, odwb), (dwl, odwl), (dsc, odsc)):
            assert rel_err(to_f64(g), o) <= TOL["f32"]


# planes that 2^L does not divide: odd band grids at one or more levels,
# down to a 1 x 1 plane analysed five times
ODD = [(2, 3, 13, 11, 2, 5, 3), (1, 2, 7, 9, 3, 3, 5), (2, 4, 57, 45, 3, 5, 5), (1, 3, 1, 1, 5, 3, 3),
       (1, 2, 100, 3, 4, 7, 7), (1, 2, 129, 255, 5, 5, 5)]


@pytest.mark.parametrize("shape", ODD + [(2, 3, 28, 28, 2, 9, 9), (1, 4, 20, 24, 2, 1, 3), (1, 2, 33, 30, 3, 3, 15)],
                         ids=lambda s: "x".join(map(str, s)))
def test_odd_planes_match_oracle(shape):
    """Forward, backward data and backward weight on planes that 2^L does
    not divide, and with kernels the fused plans do not cover (1, 9, 15),
    fp32 and bf16, against the oracle."""
    _say(f"[parity] odd plane {shape}")
    _check_all_three(*shape, seed=17)


@pytest.mark.parametrize("shape", [(2, 3, 56, 56, 3, 5, 5), (2, 3, 64, 64, 4, 3, 3), (1, 2, 256, 256, 4, 7, 5),
                                   (3, 70, 14, 14, 1, 5, 5), (1, 4, 13, 11, 2, 3, 5), (2, 2, 28, 28, 0, 7, 3)],
                         ids=lambda s: "x".join(map(str, s)))
def test_channels_last_matches_oracle(shape):
    """Channels-last activations give the oracle's results, and y and dx come
    back channels last. Planned shapes (whole-plane, split, large-plane
    tiles; 70 channels leave a partial 64-channel tile) run the planar
    kernels on converted copies and must equal the planar call bit for bit;
    the others run the generic chain."""
    _say(f"[parity] channels last {shape}")
    cl = torch.channels_last
    for dtype in ("f32", "bf16"):
        inp = make_inputs(*shape, dtype=dtype, seed=19)
        x, dy, wb, wl, sc = to_device(inp)
        x, dy = x.contiguous(memory_format=cl), dy.contiguous(memory_format=cl)
        assert not x.is_contiguous()
        y = wt.wtconv_fwd(x, wb, wl, sc)
        dx = wt.wtconv_bwd_data(dy, wb, wl, sc)
        dwb, dwl, dsc = wt.wtconv_bwd_weight(x, dy, shape[5], wl, sc)
        torch.cuda.synchronize()
        assert y.is_contiguous(memory_format=cl) and dx.is_contiguous(memory_format=cl)
        oy, odx, (odwb, odwl, odsc) = _oracle_all(inp)
        assert rel_err(to_f64(y), oy) <= TOL[dtype] and rel_err(to_f64(dx), odx) <= TOL[dtype]
        for g, o in ((dwb, odwb), (dwl, odwl), (dsc, odsc)):
            if g.numel():
                assert rel_err(to_f64(g), o) <= TOL["f32"]
        if shape[4] > 0 and shape[2] % (1 << shape[4]) == 0:
            xp, dyp = x.contiguous(), dy.contiguous()
            planar = (wt.wtconv_fwd(xp, wb, wl, sc), wt.wtconv_bwd_data(dyp, wb, wl, sc),
                      *wt.wtconv_bwd_weight(xp, dyp, shape[5], wl, sc))
            torch.cuda.synchronize()
            for a, b in zip((y, dx, dwb, dwl, dsc), planar):
                assert torch.equal(a.contiguous(), b)


def test_hand_worked_odd_plane_on_gpu():
    """The hand-worked 3x3 example (tests/golden) through the C-ABI: values
    fixed by hand, not by the oracle."""
    import json
    import os
    _say("[parity] hand-worked 3x3 odd plane")
    with open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked_3x3_odd_l1.json")) as f:
        g = json.load(f)
    dev = "cuda"
    x = torch.tensor(g["x"], dtype=torch.float32, device=dev)[None, None].contiguous()
    wb = torch.ones(1, 1, 1, device=dev)
    wl = torch.ones(1, 1, 4, 1, 1, device=dev)
    for key in ("case_ll_only", "case_band3"):
        sc = torch.tensor(g[key]["scale"], dtype=torch.float32, device=dev)[None, None].contiguous()
        y = wt.wtconv_fwd(x, wb, wl, sc)
        torch.cuda.synchronize()
        assert rel_err(to_f64(y[0, 0]), np.array(g[key]["y"])) <= 1e-6, key
    imp = g["case_band3"]["dy_impulse_2_2"]
    dy = torch.tensor(imp["dy"], dtype=torch.float32, device=dev)[None, None].contiguous()
    dx = wt.wtconv_bwd_data(dy, wb, wl, sc)
    dwb, dwl, dsc = wt.wtconv_bwd_weight(x, dy, 1, wl, sc)
    torch.cuda.synchronize()
    assert rel_err(to_f64(dx[0, 0]), np.array(imp["dx"])) <= 1e-6
    assert abs(float(dwb.flatten()[0]) - imp["dw_base"]) <= 1e-5
    assert rel_err(to_f64(dwl[0, 0, :, 0, 0]), np.array(imp["dw_lvl"])) <= 1e-6
    assert rel_err(to_f64(dsc[0, 0]), np.array(imp["dscale"])) <= 1e-6


def _random_cases(n, seed=2024):
    """Seeded small shapes over every route: planned and unplanned planes,
    odd band grids, L 0..5, odd kernels 1..9, both layouts."""
    rng = np.random.default_rng(seed)
    planned = [(56, 56, 3, 5, 5), (28, 28, 2, 5, 5), (14, 14, 1, 5, 5), (32, 32, 2, 5, 5), (64, 64, 4, 3, 3),
               (128, 128, 2, 5, 5), (24, 40, 3, 3, 3)]
    out = []
    for i in range(n):
        B, C = int(rng.integers(1, 4)), int(rng.integers(1, 6))
        if i % 3 == 0:
            H, W, L, kb, k = planned[int(rng.integers(len(planned)))]
        else:
            H, W = int(rng.integers(1, 40)), int(rng.integers(1, 40))
            L, kb, k = int(rng.integers(0, 6)), int(rng.choice([1, 3, 5, 7, 9])), int(rng.choice([1, 3, 5, 7, 9]))
        out.append((B, C, H, W, L, kb, k, bool(rng.integers(2)), ("f32", "bf16")[int(rng.integers(2))]))
    return out


@pytest.mark.parametrize("case", _random_cases(40), ids=lambda c: "x".join(map(str, c)))
def test_random_shapes_match_oracle(case):
    """Forty seeded random shapes through the three entry points against the
    oracle (layouts, odd grids, every level count and kernel size)."""
    B, C, H, W, L, kb, k, cl, dtype = case
    _say(f"[parity] random {case}")
    inp = make_inputs(B, C, H, W, L, kb, k, dtype=dtype, seed=31)
    x, dy, wb, wl, sc = to_device(inp)
    if cl:
        x, dy = x.contiguous(memory_format=torch.channels_last), dy.contiguous(memory_format=torch.channels_last)
    y = wt.wtconv_fwd(x, wb, wl, sc)
    dx = wt.wtconv_bwd_data(dy, wb, wl, sc)
    dwb, dwl, dsc = wt.wtconv_bwd_weight(x, dy, kb, wl, sc)
    torch.cuda.synchronize()
    oy, odx, (odwb, odwl, odsc) = _oracle_all(inp)
    assert rel_err(to_f64(y), oy) <= TOL[dtype] and rel_err(to_f64(dx), odx) <= TOL[dtype]
    for g, o in ((dwb, odwb), (dwl, odwl), (dsc, odsc)):
        if g.numel():
            assert rel_err(to_f64(g), o) <= TOL["f32"]


@pytest.mark.parametrize("shape", [(3, 4, 56, 56, 0, 5, 5), (2, 3, 56, 56, 0, 7, 5), (3, 5, 28, 28, 0, 5, 3),
                                   (1, 3, 28, 28, 0, 7, 7), (17, 3, 14, 14, 0, 5, 5), (5, 2, 14, 14, 0, 7, 3)],
                         ids=lambda s: "x".join(map(str, s)))
def test_level_zero_fused_kernels(shape):
    """L = 0 (the plain depthwise correlation) on the planes its fused
    kernels cover, with batches that leave the last group of images partial:
    against the oracle and against torch's own grouped convolution (fp64 on
    the CPU), both layouts."""
    _say(f"[parity] L = 0 fused {shape}")
    B, C, H, W, L, kb, k = shape
    for dtype in ("f32", "bf16"):
        inp = make_inputs(*shape, dtype=dtype, seed=41)
        x, dy, wb, wl, sc = to_device(inp)
        oy, odx, (odwb, _, _) = _oracle_all(inp)
        xd = torch.from_numpy(inp.act_f64("x"))
        ref = torch.nn.functional.conv2d(xd, torch.from_numpy(inp.params_f64()[0])[:, None], padding=kb // 2,
                                         groups=C).numpy()
        for fmt in (torch.contiguous_format, torch.channels_last):
            xi, dyi = x.contiguous(memory_format=fmt), dy.contiguous(memory_format=fmt)
            y = wt.wtconv_fwd(xi, wb, wl, sc)
            dx = wt.wtconv_bwd_data(dyi, wb, wl, sc)
            dwb, _, _ = wt.wtconv_bwd_weight(xi, dyi, kb, wl, sc)
            torch.cuda.synchronize()
            assert rel_err(to_f64(y), oy) <= TOL[dtype] and rel_err(to_f64(y), ref) <= TOL[dtype]
            assert rel_err(to_f64(dx), odx) <= TOL[dtype]
            assert rel_err(to_f64(dwb), odwb) <= TOL["f32"]


@pytest.mark.parametrize("shape", [(3, 4, 56, 56, 0, 5, 5), (2, 3, 56, 56, 0, 7, 5), (5, 3, 28, 28, 0, 7, 5),
                                   (4, 3, 28, 28, 0, 5, 5), (17, 3, 14, 14, 0, 5, 5), (5, 2, 14, 14, 0, 7, 3),
                                   (2, 3, 56, 56, 3, 5, 5), (2, 3, 13, 11, 2, 5, 3),
                                   # whole planes: the weight gradient's second stage in the data kernel's launch
                                   (11, 3, 14, 14, 1, 5, 5), (3, 2, 28, 28, 2, 5, 5), (2, 3, 128, 128, 3, 5, 5),
                                   (2, 2, 56, 56, 2, 7, 3), (3, 2, 7, 7, 2, 5, 7),
                                   # split planes: the data pass's coarse step reads the weight pass's dy sums
                                   (2, 3, 64, 64, 4, 3, 3), (3, 2, 64, 64, 2, 5, 5), (1, 2, 256, 256, 4, 7, 5),
                                   (3, 5, 256, 256, 4, 7, 5),
                                   # one-level single pass (14x14, 5x5): one image per chunk with three
                                   # idle planes per step; chunks of several steps, the last one partial
                                   (30, 200, 14, 14, 1, 5, 5), (64, 384, 14, 14, 1, 5, 5)],
                         ids=lambda s: "x".join(map(str, s)))
def test_whole_backward_equals_the_two_calls(shape):
    """wtconv_bwd (a single pass over x and dy at L = 0 on planned planes
    and at L = 1 on the 14x14 plane with 5x5 kernels; on split planes the
    weight pass first and the data pass's coarse step on its dy sums; on
    whole planes the weight pass first and its second stage in the data
    kernel's launch; the two calls elsewhere) equals wtconv_bwd_data +
    wtconv_bwd_weight bit for bit, except that the one-level single pass
    groups the tap products differently (its weight gradients agree with
    the two calls to fp32 rounding, its dx bit for bit); every form matches
    the oracle within the bars and repeats bit for bit."""
    _say(f"[parity] whole backward {shape}")
    kb = shape[5]
    one_level_pass = shape[2:] == (14, 14, 1, 5, 5)
    for dtype in ("f32", "bf16"):
        inp = make_inputs(*shape, dtype=dtype, seed=43)
        x, dy, wb, wl, sc = to_device(inp)
        dx, (dwb, dwl, dsc) = wt.wtconv_bwd(x, dy, wb, wl, sc)
        dx2 = wt.wtconv_bwd_data(dy, wb, wl, sc)
        dwb2, dwl2, dsc2 = wt.wtconv_bwd_weight(x, dy, kb, wl, sc)
        dx3, (dwb3, dwl3, dsc3) = wt.wtconv_bwd(x, dy, wb, wl, sc)
        torch.cuda.synchronize()
        assert torch.equal(dx, dx2)
        for a, b, c in ((dwb, dwb2, dwb3), (dwl, dwl2, dwl3), (dsc, dsc2, dsc3)):
            assert torch.equal(a, c)   # deterministic
            if one_level_pass:
                assert rel_err(to_f64(a), to_f64(b)) <= 1e-5
            else:
                assert torch.equal(a, b)
        assert torch.equal(dx, dx3)
        _, odx, (odwb, odwl, odsc) = _oracle_all(inp)
        assert rel_err(to_f64(dx), odx) <= TOL[dtype] and rel_err(to_f64(dwb), odwb) <= TOL["f32"]
        if shape[4] > 0:
            assert rel_err(to_f64(dwl), odwl) <= TOL["f32"] and rel_err(to_f64(dsc), odsc) <= TOL["f32"]


def test_empty_batch():
    """B = 0: empty outputs from the data passes and zero weight gradients
    (every output element overwritten)."""
    _say("[parity] empty batch")
    inp = make_inputs(1, 3, 56, 56, 3, 5, 5, dtype="bf16", seed=3)
    x, dy, wb, wl, sc = to_device(inp)
    x0, dy0 = x[:0], dy[:0]
    assert wt.wtconv_fwd(x0, wb, wl, sc).shape == (0, 3, 56, 56)
    assert wt.wtconv_bwd_data(dy0, wb, wl, sc).shape == (0, 3, 56, 56)
    out = tuple(torch.full(s, float("nan"), device="cuda") for s in ((3, 5, 5), tuple(wl.shape), tuple(sc.shape)))
    wt.wtconv_bwd_weight(x0, dy0, 5, wl, sc, out=out)
    torch.cuda.synchronize()
    assert all(bool((g == 0).all()) for g in out)


@pytest.mark.parametrize("shape", [(4, 3, 56, 56, 3, 5, 5), (2, 3, 64, 64, 4, 3, 3), (2, 3, 13, 11, 2, 5, 3)],
                         ids=lambda s: "x".join(map(str, s)))
def test_graph_replay_matches_eager(shape):
    """The three calls captured in one HIP graph (whole-plane, split and
    generic-chain shapes): every replay, with other eager work and
    synchronisation between replays, equals the eager results bit for bit
    (the kernels are deterministic and the library records no memset)."""
    _say(f"[parity] graph replay {shape}")
    B, C, H, W, L, kb, k = shape
    inp = make_inputs(*shape, dtype="bf16", seed=23)
    x, dy, wb, wl, sc = to_device(inp)
    ws = torch.empty(max(wt.wtconv_workspace_size(x, L, kb, k, op) for op in range(3)) + 256, dtype=torch.uint8,
                     device="cuda")
    y, dx = torch.empty_like(x), torch.empty_like(x)
    gr = (torch.empty(C, kb, kb, device="cuda"), torch.empty(tuple(wl.shape), device="cuda"),
          torch.empty(tuple(sc.shape), device="cuda"))

    def step():
        wt.wtconv_fwd(x, wb, wl, sc, y=y, ws=ws)
        wt.wtconv_bwd_data(dy, wb, wl, sc, dx=dx, ws=ws)
        wt.wtconv_bwd_weight(x, dy, kb, wl, sc, out=gr, ws=ws)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (y, dx, *gr)]
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for r in range(3):
        for t in (y, dx, *gr):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip((y, dx, *gr), eager):
            assert torch.equal(t, e), f"replay {r}"
        (x.float() * 2).sum().item()   # eager work between replays


@pytest.mark.parametrize("shape", [(24, 16, 14, 14, 1, 5, 5), (4, 3, 56, 56, 3, 5, 5), (2, 3, 64, 64, 4, 3, 3)],
                         ids=lambda s: "x".join(map(str, s)))
def test_graph_replay_whole_backward(shape):
    """wtconv_bwd captured in a HIP graph (the one-level single pass with its
    second-stage launch, the weight pass with its second stage in the data
    kernel's launch, the split plane's shared dy sums): every replay, with
    eager work between replays, equals the eager result bit for bit."""
    _say(f"[parity] graph replay of the whole backward {shape}")
    B, C, H, W, L, kb, k = shape
    inp = make_inputs(*shape, dtype="bf16", seed=29)
    x, dy, wb, wl, sc = to_device(inp)
    ws = torch.empty(wt.wtconv_workspace_size(x, L, kb, k, 3) + 256, dtype=torch.uint8, device="cuda")
    dx = torch.empty_like(x)
    gr = (torch.empty(C, kb, kb, device="cuda"), torch.empty(tuple(wl.shape), device="cuda"),
          torch.empty(tuple(sc.shape), device="cuda"))

    def step():
        wt.wtconv_bwd(x, dy, wb, wl, sc, dx=dx, out=gr, ws=ws)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (dx, *gr)]
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for r in range(3):
        for t in (dx, *gr):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip((dx, *gr), eager):
            assert torch.equal(t, e), f"replay {r}"
        (x.float() * 2).sum().item()   # eager work between replays


@pytest.mark.parametrize("L", [2, 4])
def test_persistent_column_kernel_uneven_share(L):
    """The 128x128 column kernel with persistent workgroups (one per CU,
    every 256th plane each, the next plane's loads in flight): 300 planes,
    so some workgroups take two planes and the rest one; y, dx and the
    whole backward against the oracle, bf16 activations."""
    B, C, H, W, kb, k = 3, 100, 128, 128, 5, 5
    _say(f"[parity] persistent column kernel {B}x{C}x{H}x{W} L{L}")
    inp = make_inputs(B, C, H, W, L, kb, k, dtype="bf16", seed=31 + L)
    x, dy, wb, wl, sc = to_device(inp)
    y = wt.wtconv_fwd(x, wb, wl, sc)
    dx = wt.wtconv_bwd_data(dy, wb, wl, sc)
    dx1, (gb, gl, gs) = wt.wtconv_bwd(x, dy, wb, wl, sc)
    torch.cuda.synchronize()
    oy, odx, (ob, ol, os_) = _oracle_all(inp)
    assert rel_err(to_f64(y), oy) <= TOL["bf16"]
    assert rel_err(to_f64(dx), odx) <= TOL["bf16"] and torch.equal(dx, dx1)
    for g, o in ((gb, ob), (gl, ol), (gs, os_)):
        assert rel_err(to_f64(g), o) <= TOL["f32"]


def test_measurement_probes():
    """The copy probe copies exactly; the FMA probe writes finite values to
    every lane's slot; bad arguments are refused before any launch."""
    _say("[probes] copy and fma")
    src = torch.randn(1 << 20, device="cuda")
    dst = torch.full_like(src, float("nan"))
    assert wt.wtconv_peak_copy(src, dst) == 2 * src.numel() * 4
    out = torch.full((4 * 256,), float("nan"), device="cuda")
    assert wt.wtconv_peak_fma(out, 4, 100) == 2 * 16 * 100 * 256 * 4
    torch.cuda.synchronize()
    assert torch.equal(src, dst) and bool(torch.isfinite(out).all())
    with pytest.raises(wt.WTConvError):
        wt.wtconv_peak_fma(out, 0, 10)
    with pytest.raises(wt.WTConvError):
        wt.wtconv_peak_copy(src[1:5], dst[:4])   # 4-byte offset: misaligned


def test_repeated_calls_with_changing_batch():
    """Two calls in a row, the second with a smaller batch: no state is kept
    between calls."""
    _say("[parity] changing batch")
    for B in (4, 1):
        inp = make_inputs(B, 3, 56, 56, 3, dtype="f32", seed=8 + B)
        x, dy, wb, wl, sc = to_device(inp)
        y = wt.wtconv_fwd(x, wb, wl, sc)
        dwb, dwl, dsc = wt.wtconv_bwd_weight(x, dy, 5, wl, sc)
        torch.cuda.synchronize()
        oy, _, (odwb, odwl, odsc) = _oracle_all(inp)
        assert rel_err(to_f64(y), oy) <= 1e-4
        assert rel_err(to_f64(dwl), odwl) <= 1e-4 and rel_err(to_f64(dsc), odsc) <= 1e-4
