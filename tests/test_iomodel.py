"""The analytic I/O and arithmetic model (no GPU).

Pinned by counting: the multiply-adds of a call are enumerated level by level
over the actual band grids, the minimum bytes are the tensors each call must
touch, and the level sum has the closed form of a geometric series."""
import pytest

from wavelet_convolution_amd import iomodel
from wavelet_convolution_amd.configs import CONFIGS


@pytest.mark.parametrize("L,expect", [(0, 0.0), (1, 1.0), (2, 1.25), (3, 1.3125), (4, 1.328125), (5, 1.33203125)])
def test_level_sum_closed_form(L, expect):
    assert iomodel.s_levels(L) == expect
    assert abs(iomodel.s_levels(L) - 4.0 / 3.0 * (1.0 - 4.0 ** -L)) < 1e-15


@pytest.mark.parametrize("name", list(CONFIGS))
def test_macs_equal_an_enumeration_over_the_band_grids(name):
    """Per call: k_b^2 per pixel for the base, then k^2 per coefficient of
    each of the four bands at every level (band grid H/2^l x W/2^l)."""
    c = CONFIGS[name]
    count = c.B * c.C * c.H * c.W * c.kb * c.kb
    for l in range(1, c.L + 1):
        count += c.B * c.C * 4 * (c.H >> l) * (c.W >> l) * c.k * c.k
    m = iomodel.step_model(c.B, c.C, c.H, c.W, c.L, c.kb, c.k, c.dtype)
    assert m.mac_per_call == count
    assert m.flops_per_call == 2 * count and m.step_flops == 6 * count


@pytest.mark.parametrize("name", list(CONFIGS))
def test_minimum_bytes_are_the_tensors_each_call_touches(name):
    c = CONFIGS[name]
    e = 2 if c.dtype == "bf16" else 4
    act = c.B * c.C * c.H * c.W * e
    params = 4 * (c.C * c.kb * c.kb + c.L * c.C * 4 * c.k * c.k + c.L * c.C * 4)
    m = iomodel.step_model(c.B, c.C, c.H, c.W, c.L, c.kb, c.k, c.dtype)
    assert m.fwd_bytes == 2 * act + params            # x in, y out
    assert m.bwd_data_bytes == 2 * act + params       # dy in, dx out
    assert m.bwd_weight_bytes == 2 * act + 2 * params  # x and dy in, gradients out
    assert m.step_bytes == 6 * act + 4 * params
    # forward + one backward call: x read twice, dy once, y and dx written once
    assert m.step_bytes_fused_bwd == 5 * act + 3 * params


def test_stage1_figures():
    """The stage-1 shape's headline figures: 19,267,584 activations, 57.8125
    multiply-adds per activation and call, 231.7 MB minimum per step."""
    c = CONFIGS["stage1_56"]
    m = iomodel.step_model(c.B, c.C, c.H, c.W, c.L, c.kb, c.k, c.dtype)
    assert m.N == 19_267_584
    assert m.mac_per_call / m.N == 57.8125
    assert abs(m.step_bytes / 1e6 - 231.7) < 0.1


def test_naive_model_exceeds_the_minimum():
    """The unfused chain moves several times the forward minimum: every level
    writes and rereads its bands, convolution outputs and synthesis."""
    c = CONFIGS["stage1_56"]
    m = iomodel.step_model(c.B, c.C, c.H, c.W, c.L, c.kb, c.k, c.dtype)
    naive = iomodel.naive_fwd_bytes(c.B, c.C, c.H, c.W, c.L, c.dtype)
    assert naive > 5 * (m.fwd_bytes - m.param_bytes)
