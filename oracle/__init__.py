"""fp64 CPU oracle for the WTConv layer. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It never imports the HIP package and
shares no code with it; the two meet only through the seeded inputs.

The arithmetic lives in ``wtconv_oracle.c`` (plain fp64 loop nests; see its
header for the definition of the layer and the readings it takes). This
module compiles it with gcc on first use and marshals numpy arrays.

The layer follows the abstract of "I/O-aware reformulation of wavelet
convolution" (arXiv:2608.10805): a depthwise base convolution plus an
L-level Haar branch with per-(level, channel, band) convolutions and scales,
recombined by the inverse-Haar synthesis cascade.

Every function takes fp64 numpy arrays in these layouts:
    x, dy        [B, C, H, W]
    w_base       [C, kb, kb]
    w_lvl        [L, C, 4, k, k]
    scale        [L, C, 4]
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wtconv_oracle.c")
_LIB = os.path.join(_HERE, "libwtconv_oracle.so")
_lock = threading.Lock()
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.c_int


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-ffp-contract=off", "-fno-fast-math", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            dims = [_I] * 7
            for name in ("wto_fwd", "wto_fwd_closed"):
                getattr(lib, name).argtypes = dims + [_D, _D, _D, _D, _D]
            lib.wto_bwd_data.argtypes = dims + [_D, _D, _D, _D, _D]
            for name in ("wto_bwd_weight", "wto_bwd_weight_gcorr"):
                getattr(lib, name).argtypes = dims + [_D, _D, _D, _D, _D, _D, _D]
            lib.wto_haar_dwt.argtypes = [_D, _I, _I, _D]
            lib.wto_haar_iwt.argtypes = [_D, _I, _I, _D]
            lib.wto_set_threads.argtypes = [_I]
            lib.wto_max_threads.restype = _I
            _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(_D)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _dims(x, w_base, w_lvl, scale):
    B, C, H, W = x.shape
    L = w_lvl.shape[0]
    kb = w_base.shape[-1]
    k = w_lvl.shape[-1] if L > 0 else 1
    assert w_base.shape == (C, kb, kb), w_base.shape
    assert w_lvl.shape[:3] == (L, C, 4) or L == 0, w_lvl.shape
    assert scale.shape == (L, C, 4), scale.shape
    assert kb % 2 == 1 and k % 2 == 1
    assert 0 <= L <= 32 and H >= 1 and W >= 1
    return B, C, H, W, L, kb, k


def set_threads(n: int) -> None:
    """Set the OpenMP thread count used by the oracle."""
    _load().wto_set_threads(int(n))


def max_threads() -> int:
    return int(_load().wto_max_threads())


def haar_dwt(X) -> np.ndarray:
    """One orthonormal 2x2 Haar analysis step: [H, W] -> [4, ceil(H/2), ceil(W/2)].

    An odd last row or column is paired with a zero one (the odd-grid reading
    the layer takes), so the bands are ceil-sized; that is also the size the C
    routine writes."""
    X = _f64(X)
    if X.ndim != 2 or X.shape[0] < 1 or X.shape[1] < 1:
        raise ValueError(f"haar_dwt takes a non-empty 2-D plane, got shape {X.shape}")
    H, W = X.shape
    out = np.zeros((4, (H + 1) // 2, (W + 1) // 2))
    _load().wto_haar_dwt(_p(X), H, W, _p(out))
    return out


def haar_iwt(bands, shape=None) -> np.ndarray:
    """Inverse of haar_dwt: [4, h, w] -> [2h, 2w], or the top-left
    shape = (H, W) of it (H in {2h-1, 2h}, W in {2w-1, 2w}): the crop back to
    an odd plane that haar_dwt analysed."""
    bands = _f64(bands)
    if bands.ndim != 3 or bands.shape[0] != 4:
        raise ValueError(f"haar_iwt takes [4, h, w] bands, got shape {bands.shape}")
    _, h, w = bands.shape
    H, W = (2 * h, 2 * w) if shape is None else (int(shape[0]), int(shape[1]))
    if not (2 * h - 1 <= H <= 2 * h and 2 * w - 1 <= W <= 2 * w):
        raise ValueError(f"crop {H}x{W} does not fit bands of {h}x{w}")
    out = np.zeros((2 * h, 2 * w))
    _load().wto_haar_iwt(_p(bands), h, w, _p(out))
    return np.ascontiguousarray(out[:H, :W])


def _fwd_like(fn_name, x, w_base, w_lvl, scale):
    x, w_base, w_lvl, scale = map(_f64, (x, w_base, w_lvl, scale))
    B, C, H, W, L, kb, k = _dims(x, w_base, w_lvl, scale)
    y = np.zeros_like(x)
    getattr(_load(), fn_name)(B, C, H, W, L, kb, k, _p(x), _p(w_base), _p(w_lvl),
                              _p(scale), _p(y))
    return y


def fwd(x, w_base, w_lvl, scale) -> np.ndarray:
    """y = WTConv(x): the synthesis cascade, step by step."""
    return _fwd_like("wto_fwd", x, w_base, w_lvl, scale)


def fwd_closed(x, w_base, w_lvl, scale) -> np.ndarray:
    """y = WTConv(x) by the single-pass closed form (abstract, reformulation 2)."""
    return _fwd_like("wto_fwd_closed", x, w_base, w_lvl, scale)


def bwd_data(dy, w_base, w_lvl, scale) -> np.ndarray:
    """dx = J^T dy by literal reverse-mode of the cascade."""
    return _fwd_like("wto_bwd_data", dy, w_base, w_lvl, scale)


def _bwd_w(fn_name, x, dy, w_base, w_lvl, scale):
    x, dy, w_base, w_lvl, scale = map(_f64, (x, dy, w_base, w_lvl, scale))
    assert x.shape == dy.shape
    B, C, H, W, L, kb, k = _dims(x, w_base, w_lvl, scale)
    dwb = np.zeros((C, kb, kb))
    dwl = np.zeros((L, C, 4, k, k))
    dsc = np.zeros((L, C, 4))
    getattr(_load(), fn_name)(B, C, H, W, L, kb, k, _p(x), _p(dy), _p(w_lvl),
                              _p(scale), _p(dwb), _p(dwl), _p(dsc))
    return dwb, dwl, dsc


def bwd_weight(x, dy, w_base, w_lvl, scale):
    """(dW_base, dW_lvl, dscale) by literal reverse-mode of the cascade.

    w_base is taken only for its shape (the gradients do not depend on it)."""
    return _bwd_w("wto_bwd_weight", x, dy, w_base, w_lvl, scale)


def bwd_weight_gcorr(x, dy, w_base, w_lvl, scale):
    """Same gradients from the unscaled pyramid correlation G:
    dW_lvl = scale * G, dscale = sum(W * G) (abstract, reformulation 3)."""
    return _bwd_w("wto_bwd_weight_gcorr", x, dy, w_base, w_lvl, scale)
