"""Thin ctypes binding of libwtconv.so (argument marshalling only).

Every function takes torch tensors on the GPU, checks what the plain pointers
of the C ABI cannot carry (device, shape, dtype and memory order of every
tensor it passes), and calls the C-ABI entry point of the same name on the
current stream. Validation and every step of the computation
happen in the library. The library must exist: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwtconv.so")
_lock = threading.Lock()
_lib = None

WTCONV_F32, WTCONV_BF16 = 0, 1
WTCONV_NCHW, WTCONV_NHWC = 0, 1
OP_FWD, OP_BWD_DATA, OP_BWD_WEIGHT, OP_BWD = 0, 1, 2, 3


class WTConvError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class WTConvDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("C", ctypes.c_int32), ("H", ctypes.c_int32),
                ("W", ctypes.c_int32), ("levels", ctypes.c_int32), ("k_base", ctypes.c_int32),
                ("k_level", ctypes.c_int32), ("dtype", ctypes.c_int32), ("layout", ctypes.c_int32)]


_V = ctypes.c_void_p
_SZ = ctypes.c_size_t
_P = ctypes.POINTER(WTConvDesc)


def load_library() -> ctypes.CDLL:
    """Load libwtconv.so (after torch, so both share one HIP runtime)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise ImportError(
                    f"{_LIB_PATH} is missing: build it with `python -m wavelet_convolution_amd.build` "
                    "(there is no CPU fallback)")
            lib = ctypes.CDLL(_LIB_PATH)
            lib.wtconv_workspace_size.argtypes = [_P, ctypes.c_int32]
            lib.wtconv_workspace_size.restype = _SZ
            lib.wtconv_route.argtypes = [_P, ctypes.c_int32]
            lib.wtconv_route.restype = ctypes.c_int32
            lib.wtconv_naive_workspace_size.argtypes = [_P, ctypes.c_int32]
            lib.wtconv_naive_workspace_size.restype = _SZ
            for name in ("wtconv_fwd", "wtconv_bwd_data", "wtconv_naive_fwd", "wtconv_naive_bwd_data"):
                fn = getattr(lib, name)
                fn.argtypes = [_P, _V, _V, _V, _V, _V, _V, _SZ, _V]
                fn.restype = ctypes.c_int
            for name in ("wtconv_bwd_weight", "wtconv_naive_bwd_weight"):
                fn = getattr(lib, name)
                fn.argtypes = [_P, _V, _V, _V, _V, _V, _V, _V, _V, _SZ, _V]
                fn.restype = ctypes.c_int
            lib.wtconv_bwd_weight_noalloc.argtypes = [_P, _V, _V, _V, _V, _V, _V, _V, _V]
            lib.wtconv_bwd_weight_noalloc.restype = ctypes.c_int
            lib.wtconv_bwd.argtypes = [_P, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _SZ, _V]
            lib.wtconv_bwd.restype = ctypes.c_int
            lib.wtconv_peak_fma.argtypes = [_V, ctypes.c_int32, ctypes.c_int32, _V]
            lib.wtconv_peak_fma.restype = ctypes.c_int
            lib.wtconv_peak_copy.argtypes = [_V, _V, _SZ, _V]
            lib.wtconv_peak_copy.restype = ctypes.c_int
            lib.wtconv_status_string.argtypes = [ctypes.c_int]
            lib.wtconv_status_string.restype = ctypes.c_char_p
            lib.wtconv_version.restype = ctypes.c_char_p
            _lib = lib
    return _lib


def wtconv_status_string(status: int) -> str:
    return load_library().wtconv_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != 0:
        raise WTConvError(status, wtconv_status_string(status))


def layout_of(act: torch.Tensor) -> int:
    """The library's layout code for a [B, C, H, W] tensor's memory order:
    planar (contiguous) or channels last. Any other strides are an error."""
    if act.is_contiguous():
        return WTCONV_NCHW
    if act.dim() == 4 and act.is_contiguous(memory_format=torch.channels_last):
        return WTCONV_NHWC
    raise ValueError("activations must be contiguous in NCHW or channels-last order")


def _desc(act: torch.Tensor, levels: int, k_base: int, k_level: int) -> WTConvDesc:
    B, C, H, W = act.shape
    dt = {torch.float32: WTCONV_F32, torch.bfloat16: WTCONV_BF16}.get(act.dtype, -1)
    return WTConvDesc(B, C, H, W, int(levels), int(k_base), int(k_level), dt, layout_of(act))


def _same_layout(a: torch.Tensor, b: torch.Tensor) -> None:
    if b.shape != a.shape or b.dtype != a.dtype or layout_of(b) != layout_of(a):
        raise ValueError("activation tensors of one call must share shape, dtype and memory order")


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _require_gpu(act: torch.Tensor, **tensors) -> None:
    """Every pointer handed to the library must be device memory on the
    activation's GPU: a host pointer in a kernel argument is a memory fault,
    so CPU tensors (or tensors on another device) are refused here, before
    anything else is looked at."""
    if not isinstance(act, torch.Tensor) or not act.is_cuda:
        dev = act.device if isinstance(act, torch.Tensor) else type(act).__name__
        raise ValueError(f"activations must be a GPU tensor, got one on {dev}")
    for name, t in tensors.items():
        if t is None:
            continue
        for i, u in enumerate(t if isinstance(t, (tuple, list)) else (t,)):
            if u is None:
                continue
            if not isinstance(u, torch.Tensor) or not u.is_cuda or u.device != act.device:
                where = u.device if isinstance(u, torch.Tensor) else type(u).__name__
                label = name if not isinstance(t, (tuple, list)) else f"{name}[{i}]"
                raise ValueError(f"{label} must be a tensor on {act.device} (the activations' GPU), got {where}")


def _check_f32(name: str, t, shape, like: torch.Tensor) -> None:
    """The library reads and writes parameter-shaped buffers through plain
    pointers: their shape, dtype, order and device are checked here."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != torch.float32 or not t.is_contiguous() \
            or t.device != like.device:
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)} on {like.device}; "
                         f"got {tuple(t.shape)} {t.dtype} on {t.device}")


def _check_params(act: torch.Tensor, w_base, w_lvl, scale, levels: int, kb: int, k: int) -> None:
    C = act.shape[1]
    if w_base is not None:
        _check_f32("w_base", w_base, (C, kb, kb), act)
    if levels > 0:
        _check_f32("w_lvl", w_lvl, (levels, C, 4, k, k), act)
        _check_f32("scale", scale, (levels, C, 4), act)


def _dims(w_base: torch.Tensor, w_lvl: torch.Tensor):
    levels = int(w_lvl.shape[0]) if w_lvl is not None else 0
    k_level = int(w_lvl.shape[-1]) if (w_lvl is not None and w_lvl.dim() == 5) else 3
    k_base = int(w_base.shape[-1])
    return levels, k_base, k_level


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def wtconv_workspace_size(act: torch.Tensor, levels: int, k_base: int, k_level: int, op: int,
                          naive: bool = False) -> int:
    lib = load_library()
    d = _desc(act, levels, k_base, k_level)
    fn = lib.wtconv_naive_workspace_size if naive else lib.wtconv_workspace_size
    n = fn(ctypes.byref(d), int(op))
    if n == ctypes.c_size_t(-1).value:
        raise WTConvError(2, wtconv_status_string(2))
    return int(n)


ROUTES = {0: "generic", 1: "fused", 2: "fused_copies", 3: "single_pass"}


def wtconv_route(act: torch.Tensor, levels: int, k_base: int, k_level: int, op: int) -> str:
    """How the library runs `op` for this activation tensor's shape, dtype
    and layout: "generic" (the one-kernel-per-step chain), "fused",
    "fused_copies" (fused kernels on planar copies of channels-last
    activations) or "single_pass" (wtconv_bwd: one kernel for dx and every
    weight gradient). Makes no device call."""
    lib = load_library()
    d = _desc(act, levels, k_base, k_level)
    r = lib.wtconv_route(ctypes.byref(d), int(op))
    if r < 0:
        raise WTConvError(2, wtconv_status_string(2))
    return ROUTES[r]


def _workspace(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    return torch.empty(nbytes + 256, dtype=torch.uint8, device=device)


def _ws_bytes(ws: torch.Tensor | None) -> int:
    """Usable bytes of a workspace tensor after aligning its start to 256."""
    if ws is None:
        return 0
    return max(0, ws.numel() * ws.element_size() - (_ws_ptr(ws) - ws.data_ptr()))


def _ws_ptr(ws: torch.Tensor | None) -> int:
    if ws is None:
        return 0
    p = ws.data_ptr()
    return (p + 255) & ~255


def _data_pass(name: str, naive: bool, op: int, act, w_base, w_lvl, scale, out, ws, stream):
    _require_gpu(act, w_base=w_base, w_lvl=w_lvl, scale=scale, out=out, ws=ws)
    lib = load_library()
    levels, kb, k = _dims(w_base, w_lvl)
    d = _desc(act, levels, kb, k)
    _check_params(act, w_base, w_lvl, scale, levels, kb, k)
    if out is None:
        out = torch.empty_like(act)   # same memory order as act
    _same_layout(act, out)
    if ws is None:
        ws = _workspace(wtconv_workspace_size(act, levels, kb, k, op, naive), act.device)
    ws_bytes = _ws_bytes(ws)
    _check(getattr(lib, name)(ctypes.byref(d), _ptr(act), _ptr(w_base), _ptr(w_lvl), _ptr(scale),
                              _ptr(out), _ws_ptr(ws), ws_bytes, _stream(stream)))
    return out


def wtconv_fwd(x, w_base, w_lvl, scale, y=None, ws=None, stream=None):
    """y = WTConv(x). x: [B,C,H,W] fp32/bf16 CUDA tensor; w_base [C,kb,kb],
    w_lvl [L,C,4,k,k], scale [L,C,4] fp32."""
    return _data_pass("wtconv_fwd", False, OP_FWD, x, w_base, w_lvl, scale, y, ws, stream)


def wtconv_bwd_data(dy, w_base, w_lvl, scale, dx=None, ws=None, stream=None):
    """dx = J^T dy."""
    return _data_pass("wtconv_bwd_data", False, OP_BWD_DATA, dy, w_base, w_lvl, scale, dx, ws, stream)


def wtconv_naive_fwd(x, w_base, w_lvl, scale, y=None, ws=None, stream=None):
    return _data_pass("wtconv_naive_fwd", True, OP_FWD, x, w_base, w_lvl, scale, y, ws, stream)


def wtconv_naive_bwd_data(dy, w_base, w_lvl, scale, dx=None, ws=None, stream=None):
    return _data_pass("wtconv_naive_bwd_data", True, OP_BWD_DATA, dy, w_base, w_lvl, scale, dx, ws, stream)


def _bwd_weight(name: str, naive: bool, x, dy, w_base_shape_kb, w_lvl, scale, out, ws, stream):
    _require_gpu(x, dy=dy, w_lvl=w_lvl, scale=scale, out=out, ws=ws)
    lib = load_library()
    levels = int(w_lvl.shape[0])
    k = int(w_lvl.shape[-1])
    kb = int(w_base_shape_kb)
    d = _desc(x, levels, kb, k)
    _same_layout(x, dy)
    _check_params(x, None, w_lvl, scale, levels, kb, k)
    C = x.shape[1]
    if out is None:
        dev = x.device
        out = (torch.empty((C, kb, kb), dtype=torch.float32, device=dev),
               torch.empty((levels, C, 4, k, k), dtype=torch.float32, device=dev),
               torch.empty((levels, C, 4), dtype=torch.float32, device=dev))
    if ws is None:
        ws = _workspace(wtconv_workspace_size(x, levels, kb, k, OP_BWD_WEIGHT, naive), x.device)
    ws_bytes = _ws_bytes(ws)
    dwb, dwl, dsc = out
    _check_f32("dw_base", dwb, (C, kb, kb), x)
    _check_f32("dw_lvl", dwl, (levels, C, 4, k, k), x)
    _check_f32("dscale", dsc, (levels, C, 4), x)
    _check(getattr(lib, name)(ctypes.byref(d), _ptr(x), _ptr(dy), _ptr(w_lvl), _ptr(scale), _ptr(dwb),
                              _ptr(dwl), _ptr(dsc), _ws_ptr(ws), ws_bytes, _stream(stream)))
    return out


def wtconv_bwd_weight(x, dy, k_base, w_lvl, scale, out=None, ws=None, stream=None):
    """(dW_base, dW_lvl, dscale) for kernels of size k_base (base) and w_lvl's."""
    return _bwd_weight("wtconv_bwd_weight", False, x, dy, k_base, w_lvl, scale, out, ws, stream)


def wtconv_bwd_weight_noalloc(x, dy, k_base, w_lvl, scale, out=None, stream=None):
    """As wtconv_bwd_weight, with the library's static scratch array instead
    of a workspace (the C entry point allocates nothing; outputs are
    allocated here when `out` is None). Raises WTConvError
    (WTCONV_ERR_SCRATCH_LIMIT) when the call needs more than 64 MiB."""
    _require_gpu(x, dy=dy, w_lvl=w_lvl, scale=scale, out=out)
    lib = load_library()
    levels, k, kb = int(w_lvl.shape[0]), int(w_lvl.shape[-1]), int(k_base)
    d = _desc(x, levels, kb, k)
    _same_layout(x, dy)
    _check_params(x, None, w_lvl, scale, levels, kb, k)
    C = x.shape[1]
    if out is None:
        dev = x.device
        out = (torch.empty((C, kb, kb), dtype=torch.float32, device=dev),
               torch.empty((levels, C, 4, k, k), dtype=torch.float32, device=dev),
               torch.empty((levels, C, 4), dtype=torch.float32, device=dev))
    dwb, dwl, dsc = out
    _check_f32("dw_base", dwb, (C, kb, kb), x)
    _check_f32("dw_lvl", dwl, (levels, C, 4, k, k), x)
    _check_f32("dscale", dsc, (levels, C, 4), x)
    _check(lib.wtconv_bwd_weight_noalloc(ctypes.byref(d), _ptr(x), _ptr(dy), _ptr(w_lvl), _ptr(scale), _ptr(dwb),
                                         _ptr(dwl), _ptr(dsc), _stream(stream)))
    return out


def wtconv_naive_bwd_weight(x, dy, k_base, w_lvl, scale, out=None, ws=None, stream=None):
    return _bwd_weight("wtconv_naive_bwd_weight", True, x, dy, k_base, w_lvl, scale, out, ws, stream)


def wtconv_peak_fma(out: torch.Tensor, blocks: int, iters: int, stream=None) -> int:
    """Enqueue the FMA-rate probe; returns the flops it performs."""
    _require_gpu(out)
    _check(load_library().wtconv_peak_fma(_ptr(out), int(blocks), int(iters), _stream(stream)))
    return 2 * 16 * int(iters) * 256 * int(blocks)


def wtconv_peak_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> int:
    """Enqueue the copy probe over src's bytes; returns the HBM bytes moved."""
    _require_gpu(src, dst=dst)
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst is smaller than src")
    _check(load_library().wtconv_peak_copy(_ptr(src), _ptr(dst), n, _stream(stream)))
    return 2 * n


def wtconv_bwd(x, dy, w_base, w_lvl, scale, dx=None, out=None, ws=None, stream=None):
    """(dx, (dW_base, dW_lvl, dscale)) in one call: a single pass over x and
    dy where the library has one (L = 0 on its planned planes, L = 1 on
    14x14 planes with 5x5 kernels), else the library's other fused backward
    forms or the two backward calls on one workspace."""
    _require_gpu(x, dy=dy, w_base=w_base, w_lvl=w_lvl, scale=scale, dx=dx, out=out, ws=ws)
    lib = load_library()
    levels, kb, k = _dims(w_base, w_lvl)
    d = _desc(x, levels, kb, k)
    _same_layout(x, dy)
    _check_params(x, w_base, w_lvl, scale, levels, kb, k)
    C = x.shape[1]
    if dx is None:
        dx = torch.empty_like(dy)
    _same_layout(dy, dx)
    if out is None:
        dev = x.device
        out = (torch.empty((C, kb, kb), dtype=torch.float32, device=dev),
               torch.empty((levels, C, 4, k, k), dtype=torch.float32, device=dev),
               torch.empty((levels, C, 4), dtype=torch.float32, device=dev))
    dwb, dwl, dsc = out
    _check_f32("dw_base", dwb, (C, kb, kb), x)
    _check_f32("dw_lvl", dwl, (levels, C, 4, k, k), x)
    _check_f32("dscale", dsc, (levels, C, 4), x)
    if ws is None:
        ws = _workspace(wtconv_workspace_size(x, levels, kb, k, OP_BWD), x.device)
    _check(lib.wtconv_bwd(ctypes.byref(d), _ptr(x), _ptr(dy), _ptr(w_base), _ptr(w_lvl), _ptr(scale), _ptr(dx),
                          _ptr(dwb), _ptr(dwl), _ptr(dsc), _ws_ptr(ws), _ws_bytes(ws), _stream(stream)))
    return dx, out
