"""Shared test helpers: move seeded inputs to the GPU, compare with the oracle."""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(got, ref) -> float:
    """Normwise max relative error: max|got - ref| / max|ref|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (denom if denom > 0 else 1.0))


def elem_err(got, ref, floor: float = 1e-3) -> float:
    """Elementwise max relative error with a floor: max_i |got_i - ref_i| /
    max(|ref_i|, floor * max|ref|). Logged beside the normwise measure (it is
    not the parity bar): an error confined to small elements shows up here."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max()
    if scale == 0:
        return float(np.abs(got).max())
    return float((np.abs(got - ref) / np.maximum(np.abs(ref), floor * scale)).max())


def to_device(inp, device="cuda"):
    """(x, dy, w_base, w_lvl, scale) as torch tensors on the GPU."""
    import torch

    def act(a):
        if inp.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
        return torch.from_numpy(a.copy()).to(device)

    return (act(inp.x), act(inp.dy), torch.from_numpy(inp.w_base).to(device),
            torch.from_numpy(inp.w_lvl).to(device), torch.from_numpy(inp.scale).to(device))


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()
