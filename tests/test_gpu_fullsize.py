"""Parity at the full workload sizes, in the launch configuration the bench
times: the GPU computes whole tensors, the oracle recomputes sampled (b, c)
planes of y and dx and every gradient of sampled channels (all b)."""
import sys

import numpy as np
import pytest

import oracle
from tests._util import TOL, elem_err, rel_err, to_device, to_f64
from wavelet_convolution_amd.configs import CONFIGS
from wavelet_convolution_amd.inputs import make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from wavelet_convolution_amd import binding as wt  # noqa: E402


def _planes(B, C):
    return sorted({(0, 0), (B - 1, C - 1), (B // 2, C // 3), (B // 3, (2 * C) // 3)})


@pytest.mark.parametrize("name", list(CONFIGS))
def test_full_size_sampled(name):
    cfg = CONFIGS[name]
    print(f"[fullsize] {cfg.describe()}", flush=True)
    sys.stdout.flush()
    inp = make_inputs(cfg.B, cfg.C, cfg.H, cfg.W, cfg.L, cfg.kb, cfg.k, dtype=cfg.dtype, seed=0)
    x, dy, wb, wl, sc = to_device(inp)
    y = wt.wtconv_fwd(x, wb, wl, sc)
    dx = wt.wtconv_bwd_data(dy, wb, wl, sc)
    grads = wt.wtconv_bwd_weight(x, dy, cfg.kb, wl, sc)
    # the whole backward in one call, as the bench times it
    dx1, grads1 = wt.wtconv_bwd(x, dy, wb, wl, sc)
    torch.cuda.synchronize()
    tol = TOL[cfg.dtype]
    xw, dyw = inp.act_f64("x"), inp.act_f64("dy")
    wbf, wlf, scf = inp.params_f64()
    worst = {"y": 0.0, "dx": 0.0, "dw_base": 0.0, "dw_lvl": 0.0, "dscale": 0.0}
    worst_el = dict(worst)   # elementwise, floor 1e-3 max|o| (logged, not the bar)
    for b, c in _planes(cfg.B, cfg.C):
        pw = (wbf[c:c + 1], wlf[:, c:c + 1], scf[:, c:c + 1])
        oy = oracle.fwd(xw[b:b + 1, c:c + 1], *pw)
        odx = oracle.bwd_data(dyw[b:b + 1, c:c + 1], *pw)
        gy, gdx = to_f64(y[b:b + 1, c:c + 1]), to_f64(dx[b:b + 1, c:c + 1])
        ey, edx = rel_err(gy, oy), max(rel_err(gdx, odx), rel_err(to_f64(dx1[b:b + 1, c:c + 1]), odx))
        worst["y"], worst["dx"] = max(worst["y"], ey), max(worst["dx"], edx)
        worst_el["y"], worst_el["dx"] = max(worst_el["y"], elem_err(gy, oy)), max(worst_el["dx"], elem_err(gdx, odx))
        assert ey <= tol and edx <= tol, (b, c, ey, edx)
    dwb, dwl, dsc = (to_f64(g) for g in grads)
    dwb1, dwl1, dsc1 = (to_f64(g) for g in grads1)
    for c in sorted({0, cfg.C - 1, cfg.C // 2}):
        pw = (wbf[c:c + 1], wlf[:, c:c + 1], scf[:, c:c + 1])
        o = oracle.bwd_weight(xw[:, c:c + 1], dyw[:, c:c + 1], *pw)
        for key, got, got1, ref in (("dw_base", dwb[c:c + 1], dwb1[c:c + 1], o[0]),
                                    ("dw_lvl", dwl[:, c:c + 1], dwl1[:, c:c + 1], o[1]),
                                    ("dscale", dsc[:, c:c + 1], dsc1[:, c:c + 1], o[2])):
            if ref.size == 0:   # no levels
                continue
            e = max(rel_err(got, ref), rel_err(got1, ref))
            worst[key] = max(worst[key], e)
            worst_el[key] = max(worst_el[key], elem_err(got, ref))
            assert e <= TOL["f32"], (c, key, e)
    print(f"[fullsize] {name} max rel err: " + " ".join(f"{k} {v:.2e}" for k, v in worst.items()), flush=True)
    print(f"[fullsize] {name} elementwise (floor 1e-3 max|o|): "
          + " ".join(f"{k} {v:.2e}" for k, v in worst_el.items()), flush=True)
    # properties that hold everywhere: finite outputs
    assert torch.isfinite(y.float()).all() and torch.isfinite(dx.float()).all()
