"""The C-ABI library: it loads, exports every symbol the header declares,
and rejects bad arguments on the host before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wtconv.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wtconv_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    import torch  # noqa: F401  (load torch's HIP runtime first, as the binding does)
    from wavelet_convolution_amd import binding
    if not os.path.exists(binding._LIB_PATH):
        pytest.skip("libwtconv.so not built")
    return binding.load_library()


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("wtconv_fwd", "wtconv_bwd_data", "wtconv_bwd_weight", "wtconv_workspace_size",
              "wtconv_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def _desc(**kw):
    from wavelet_convolution_amd.binding import WTConvDesc
    d = dict(B=2, C=4, H=56, W=56, levels=3, k_base=5, k_level=5, dtype=1)
    d.update(kw)
    return WTConvDesc(**d)


def test_status_strings(lib):
    for s in range(5):
        assert lib.wtconv_status_string(s).decode().startswith("WTCONV")


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), 1), (dict(C=0), 1), (dict(C=-1), 1), (dict(W=0), 1), (dict(dtype=7), 1), (dict(layout=2), 1), (dict(layout=-1), 1),
    (dict(levels=6), 2), (dict(levels=-1), 2), (dict(k_base=4), 2), (dict(k_level=17), 2), (dict(k_base=-1), 2),
    (dict(H=1 << 16, W=1 << 15), 2),  # a plane above 2^30 elements
])
def test_bad_descriptors_rejected_before_launch(lib, kw, status):
    d = _desc(**kw)
    fake = ctypes.c_void_p(1 << 20)   # never dereferenced: validation fails first
    rc = lib.wtconv_fwd(ctypes.byref(d), fake, fake, fake, fake, ctypes.c_void_p(2 << 20), None, 0, None)
    assert rc == status


def test_null_and_misaligned_pointers_rejected(lib):
    d = _desc()
    ok = ctypes.c_void_p(1 << 20)
    assert lib.wtconv_fwd(ctypes.byref(d), None, ok, ok, ok, ok, None, 0, None) == 1
    assert lib.wtconv_fwd(ctypes.byref(d), ctypes.c_void_p((1 << 20) + 2), ok, ok, ok,
                          ctypes.c_void_p(2 << 20), None, 0, None) == 1
    # input and output overlapping
    assert lib.wtconv_fwd(ctypes.byref(d), ok, ok, ok, ok, ok, None, 0, None) == 1


def test_unplanned_plane_takes_the_generic_chain(lib):
    """A plane size without a fused kernel runs the generic chain, which
    needs a workspace: its size is reported, and a call without one is
    refused before anything launches. Planes that 2^L does not divide (odd
    band grids) take it too."""
    d = _desc(H=40, W=48, levels=3)
    ok = ctypes.c_void_p(1 << 20)
    for op in (0, 1, 2):
        assert 0 < lib.wtconv_workspace_size(ctypes.byref(d), op) < (1 << 40)
    assert lib.wtconv_fwd(ctypes.byref(d), ok, ok, ok, ok, ctypes.c_void_p(1 << 30), None, 0, None) == 3
    for H, W in ((40, 44), (13, 11), (1, 1)):
        d = _desc(H=H, W=W, levels=3)
        for op in (0, 1, 2):
            assert 0 < lib.wtconv_workspace_size(ctypes.byref(d), op) < (1 << 40)
        assert lib.wtconv_fwd(ctypes.byref(d), ok, ok, ok, ok, ctypes.c_void_p(1 << 30), None, 0, None) == 3


def test_bwd_weight_workspace_checked(lib):
    d = _desc()
    need = lib.wtconv_workspace_size(ctypes.byref(d), 2)
    assert 0 < need < (1 << 40)
    ok = ctypes.c_void_p(1 << 20)
    # too small
    assert lib.wtconv_bwd_weight(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, ctypes.c_void_p(1 << 24),
                                 need - 4, None) == 3
    # misaligned
    assert lib.wtconv_bwd_weight(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, ctypes.c_void_p((1 << 24) + 16),
                                 need, None) == 3


def test_channels_last_workspace(lib):
    """A channels-last call of a planned shape runs the planar kernels on
    planar copies of its activations, which live in the workspace after the
    kernels' own part; a shape without a plan takes the generic chain."""
    def a256(n):
        return (n + 255) // 256 * 256

    planar, nhwc = _desc(layout=0), _desc(layout=1)
    act = 2 * 4 * 56 * 56 * 2   # B C H W, bf16
    assert lib.wtconv_workspace_size(ctypes.byref(planar), 0) == 0
    for op in (0, 1, 2):
        own = lib.wtconv_workspace_size(ctypes.byref(planar), op)
        assert lib.wtconv_workspace_size(ctypes.byref(nhwc), op) == a256(own) + 2 * a256(act)
    odd = _desc(H=13, W=11, layout=1)
    for op in (0, 1, 2):
        assert lib.wtconv_workspace_size(ctypes.byref(odd), op) == lib.wtconv_naive_workspace_size(
            ctypes.byref(odd), op) > 0


def test_binding_reads_the_memory_order():
    """The binding's layout code follows the tensor's strides and refuses any
    other order (a transposed view would otherwise be read as planar)."""
    import torch
    from wavelet_convolution_amd.binding import layout_of
    x = torch.zeros(2, 3, 8, 6)
    assert layout_of(x) == 0
    assert layout_of(x.to(memory_format=torch.channels_last)) == 1
    assert layout_of(torch.zeros(1, 1, 8, 6).to(memory_format=torch.channels_last)) == 0
    with pytest.raises(ValueError):
        layout_of(x.transpose(2, 3))


def test_empty_batch_is_a_no_op_for_the_data_passes(lib):
    """B = 0: the data passes validate and return without launching (the
    activation pointers may be NULL); they need no workspace. The weight
    gradient of an empty batch (zeros) runs on the GPU and is tested there."""
    d = _desc(B=0)
    ok = ctypes.c_void_p(1 << 20)
    assert lib.wtconv_workspace_size(ctypes.byref(d), 0) == 0
    assert lib.wtconv_workspace_size(ctypes.byref(d), 2) > 0
    for fn in (lib.wtconv_fwd, lib.wtconv_bwd_data, lib.wtconv_naive_fwd):
        assert fn(ctypes.byref(d), None, ok, ok, ok, None, None, 0, None) == 0
        assert fn(ctypes.byref(d), None, None, ok, ok, None, None, 0, None) == 1   # parameters still checked


def test_huge_channel_counts_leave_the_multi_image_kernels(lib):
    """The 14x14 kernel packs eight images of a channel per workgroup and
    addresses them with 32-bit offsets: with 8*C*H*W at or past 2^32 elements
    the shape takes the generic chain instead (sizes only: nothing runs)."""
    small = _desc(B=8, C=1000, H=14, W=14, levels=1)
    huge = _desc(B=8, C=1 << 22, H=14, W=14, levels=1)   # 8 * 2^22 * 196 > 2^32
    assert lib.wtconv_workspace_size(ctypes.byref(small), 0) == 0
    assert lib.wtconv_workspace_size(ctypes.byref(huge), 0) == lib.wtconv_naive_workspace_size(
        ctypes.byref(huge), 0) > 0


def test_binding_refuses_host_tensors(monkeypatch):
    """The library takes plain device pointers, so the binding refuses any CPU
    tensor it would pass (activations, parameters, outputs, gradients,
    workspace) before it even loads the library: a host pointer in a kernel
    argument would be a GPU memory fault."""
    import torch
    from wavelet_convolution_amd import binding as wt

    def no_library():
        raise AssertionError("the library must not be reached with a host tensor")

    monkeypatch.setattr(wt, "load_library", no_library)
    x = torch.zeros(1, 4, 8, 8)
    wb, wl, sc = torch.zeros(4, 5, 5), torch.zeros(1, 4, 4, 3, 3), torch.zeros(1, 4, 4)
    grads = (torch.zeros(4, 5, 5), torch.zeros(1, 4, 4, 3, 3), torch.zeros(1, 4, 4))
    ws = torch.zeros(1024, dtype=torch.uint8)
    calls = [
        lambda: wt.wtconv_fwd(x, wb, wl, sc),
        lambda: wt.wtconv_fwd(x, wb, wl, sc, y=torch.zeros_like(x)),
        lambda: wt.wtconv_fwd(x, wb, wl, sc, ws=ws),
        lambda: wt.wtconv_bwd_data(x, wb, wl, sc, dx=torch.zeros_like(x)),
        lambda: wt.wtconv_naive_fwd(x, wb, wl, sc),
        lambda: wt.wtconv_bwd_weight(x, x, 5, wl, sc, out=grads),
        lambda: wt.wtconv_bwd_weight(x, x, 5, wl, sc, ws=ws),
        lambda: wt.wtconv_naive_bwd_weight(x, x, 5, wl, sc),
        lambda: wt.wtconv_bwd(x, x, wb, wl, sc, dx=torch.zeros_like(x), out=grads, ws=ws),
        lambda: wt.wtconv_peak_fma(torch.zeros(256), 1, 1),
        lambda: wt.wtconv_peak_copy(torch.zeros(16), torch.zeros(16)),
        lambda: wt.wtconv_fwd("not a tensor", wb, wl, sc),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="GPU|activations' GPU|cuda"):
            call()


@pytest.mark.gpu
def test_binding_checks_buffers_on_the_gpu():
    """On the GPU: parameter, output and gradient buffers of the wrong shape,
    dtype, order or device are refused before the library is called, and so
    is a host tensor among GPU ones (output, workspace, dy, gradient)."""
    import torch
    from wavelet_convolution_amd import binding as wt
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda")
    x = torch.zeros(1, 4, 8, 8, device=dev)
    wb, wl, sc = (torch.zeros(4, 5, 5, device=dev), torch.zeros(1, 4, 4, 3, 3, device=dev),
                  torch.zeros(1, 4, 4, device=dev))
    bad = [(torch.zeros(3, 5, 5, device=dev), wl, sc), (wb.double(), wl, sc),
           (wb, torch.zeros(1, 4, 4, 3, 3, device=dev)[..., ::2, :], sc), (wb, wl, torch.zeros(2, 4, 4, device=dev)),
           (wb.cpu(), wl, sc)]
    for args in bad:
        with pytest.raises(ValueError):
            wt.wtconv_fwd(x, *args)
    grads = (torch.zeros(4, 5, 5, device=dev), torch.zeros(1, 4, 4, 3, 3, device=dev),
             torch.zeros(1, 4, 4, device=dev))
    with pytest.raises(ValueError):
        wt.wtconv_bwd_weight(x, x, 5, wl, sc, out=(grads[0], grads[1], torch.zeros(1, 4, 5, device=dev)))
    with pytest.raises(ValueError):
        wt.wtconv_bwd_weight(x, x, 5, wl, sc, out=(grads[0].cpu(), grads[1], grads[2]))
    with pytest.raises(ValueError):
        wt.wtconv_bwd_weight(x, x.cpu(), 5, wl, sc)
    with pytest.raises(ValueError):
        wt.wtconv_fwd(x, wb, wl, sc, y=torch.zeros(1, 4, 8, 8, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        wt.wtconv_fwd(x, wb, wl, sc, y=torch.zeros(1, 4, 8, 8))
    with pytest.raises(ValueError):
        wt.wtconv_fwd(x, wb, wl, sc, ws=torch.zeros(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        wt.wtconv_bwd(x, x, wb, wl, sc, dx=torch.zeros(1, 4, 8, 8))


def test_whole_backward_workspace(lib):
    """wtconv_bwd: the single-pass kernel's workspace where it exists (L = 0 on
    a planned plane, planar), else enough for the two backward calls."""
    for kw in (dict(levels=0), dict(levels=0, layout=1), dict(levels=3), dict(levels=2, H=13, W=11)):
        d = _desc(**kw)
        need = lib.wtconv_workspace_size(ctypes.byref(d), 3)
        parts = [lib.wtconv_workspace_size(ctypes.byref(d), op) for op in (1, 2)]
        assert 0 < need < (1 << 40)
        if kw.get("levels") == 0 and kw.get("layout", 0) == 0:
            assert need == parts[1]   # the same partial sums as the weight kernel
        else:
            assert need == max(parts)
    d = _desc(levels=0)
    ok = ctypes.c_void_p(1 << 20)
    # dx overlapping dy is refused before anything launches
    assert lib.wtconv_bwd(ctypes.byref(d), ok, ctypes.c_void_p(1 << 24), ok, ok, ok, ctypes.c_void_p(1 << 24), ok,
                          ok, ok, ctypes.c_void_p(1 << 28), 1 << 30, None) == 1


def test_route_query(lib):
    """wtconv_route tells the fused routes from the generic chain without a
    device call: the bench workloads are fused (one kernel for the whole
    backward at 14x14, L = 1 and at L = 0), channels-last calls of planned
    shapes run the fused kernels on planar copies, an unplanned shape takes
    the generic chain, and an invalid descriptor or op reports -1."""
    from wavelet_convolution_amd.binding import WTConvDesc
    from wavelet_convolution_amd.configs import CONFIGS
    for cfg in CONFIGS.values():
        d = WTConvDesc(cfg.B, cfg.C, cfg.H, cfg.W, cfg.L, cfg.kb, cfg.k, 1 if cfg.dtype == "bf16" else 0, 0)
        routes = [lib.wtconv_route(ctypes.byref(d), op) for op in (0, 1, 2, 3)]
        single = cfg.L == 0 or (cfg.H, cfg.W, cfg.L, cfg.kb, cfg.k) == (14, 14, 1, 5, 5)
        assert routes == [1, 1, 1, 3 if single else 1], (cfg.name, routes)
    d = WTConvDesc(64, 96, 56, 56, 3, 5, 5, 1, 1)   # channels last
    assert [lib.wtconv_route(ctypes.byref(d), op) for op in (0, 1, 2, 3)] == [2, 2, 2, 2]
    d = WTConvDesc(2, 3, 30, 30, 2, 5, 5, 1, 0)     # no fused kernel for 30x30
    assert [lib.wtconv_route(ctypes.byref(d), op) for op in (0, 1, 2, 3)] == [0, 0, 0, 0]
    d = WTConvDesc(0, 3, 56, 56, 3, 5, 5, 1, 0)     # empty batch
    assert lib.wtconv_route(ctypes.byref(d), 3) == 0
    d = WTConvDesc(2, 3, 56, 56, 3, 4, 5, 1, 0)     # even kernel: invalid
    assert lib.wtconv_route(ctypes.byref(d), 0) == -1
    d = WTConvDesc(2, 3, 56, 56, 3, 5, 5, 1, 0)
    assert lib.wtconv_route(ctypes.byref(d), 7) == -1
