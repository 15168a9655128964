"""The ConvNeXt stage-plane family on the fused kernels: planes of 56, 28, 14
and 7 pixels, L = 1 .. min(4, log2 H), base kernels 5 and 7, level kernels
3, 5 and 7 (the WTConvNeXt setting over decomposition levels and tensor
shapes). Planes that 2^L does not divide run zero-padded to the next
multiple of 2^L, which is the odd-grid reading of the layer.

CPU: every member is routed to fused kernels (the data passes need no
workspace, the weight gradient less than the generic chain's). GPU: every
member's forward, backward data and weight gradients against the oracle, by
the three calls and by the whole backward in one call."""
import ctypes
import os

import pytest

FAMILY = [(h, L, kb, k) for h, lmax in ((56, 4), (28, 4), (14, 3), (7, 2))
          for L in range(1, lmax + 1) for kb in (5, 7) for k in (3, 5, 7)]


def _ids(m):
    return "h{}_L{}_kb{}_k{}".format(*m)


@pytest.fixture(scope="module")
def lib():
    import torch  # noqa: F401  (torch's HIP runtime first, as the binding does)
    from wavelet_convolution_amd import binding
    if not os.path.exists(binding._LIB_PATH):
        pytest.skip("libwtconv.so not built")
    return binding.load_library()


@pytest.mark.parametrize("member", FAMILY, ids=_ids)
def test_family_routes_to_fused_kernels(lib, member):
    from wavelet_convolution_amd.binding import WTConvDesc
    h, L, kb, k = member
    for dtype in (0, 1):
        d = WTConvDesc(16, 96, h, h, L, kb, k, dtype, 0)
        for op in (0, 1):   # whole-plane data kernels keep everything on chip
            assert lib.wtconv_workspace_size(ctypes.byref(d), op) == 0, (member, dtype, op)
        fused = lib.wtconv_workspace_size(ctypes.byref(d), 2)
        naive = lib.wtconv_naive_workspace_size(ctypes.byref(d), 2)
        assert 0 < fused < naive, (member, dtype, fused, naive)
        # the route query says the same: fused data passes and weight
        # gradient; the whole backward fused (one kernel for one-level 14x14
        # planes with 5x5 kernels)
        routes = [lib.wtconv_route(ctypes.byref(d), op) for op in (0, 1, 2, 3)]
        single = (h, L, kb, k) == (14, 1, 5, 5)
        assert routes == [1, 1, 1, 3 if single else 1], (member, dtype, routes)


torch = pytest.importorskip("torch")


@pytest.mark.gpu
@pytest.mark.parametrize("member", FAMILY, ids=_ids)
def test_family_matches_oracle(member):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    from tests._util import TOL, rel_err, to_device, to_f64
    from wavelet_convolution_amd import binding as wt
    from wavelet_convolution_amd.inputs import make_inputs
    h, L, kb, k = member
    # a ragged batch for the multi-image kernels (14x14: 8 images per group)
    B, C = (3, 2) if h >= 28 else (11, 2)
    for dtype in ("f32", "bf16"):
        print(f"[family] {member} {dtype}", flush=True)
        inp = make_inputs(B, C, h, h, L, kb, k, dtype=dtype, seed=h + 10 * L + kb + k)
        x, dy, wb, wl, sc = to_device(inp)
        y = wt.wtconv_fwd(x, wb, wl, sc)
        dx = wt.wtconv_bwd_data(dy, wb, wl, sc)
        gb, gl, gs = wt.wtconv_bwd_weight(x, dy, kb, wl, sc)
        dx1, (gb1, gl1, gs1) = wt.wtconv_bwd(x, dy, wb, wl, sc)   # the whole backward in one call
        torch.cuda.synchronize()
        xo, dyo = inp.act_f64("x"), inp.act_f64("dy")
        pw = inp.params_f64()
        tol = TOL[dtype]
        assert rel_err(to_f64(y), oracle.fwd(xo, *pw)) <= tol
        odx = oracle.bwd_data(dyo, *pw)
        assert rel_err(to_f64(dx), odx) <= tol and rel_err(to_f64(dx1), odx) <= tol
        ob, ol, os_ = oracle.bwd_weight(xo, dyo, *pw)
        for got in ((gb, gl, gs), (gb1, gl1, gs1)):
            assert rel_err(to_f64(got[0]), ob) <= TOL["f32"]
            assert rel_err(to_f64(got[1]), ol) <= TOL["f32"]
            assert rel_err(to_f64(got[2]), os_) <= TOL["f32"]
