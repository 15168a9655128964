"""The seeded input generator: bf16 rounding and chunked draws."""
import numpy as np

from wavelet_convolution_amd import inputs as I


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e-3], dtype=np.float32)
    out = I.bf16_bits_to_f32(I.f32_to_bf16_bits(vals))
    # 1+2^-8 is a tie between 1 and 1+2^-7: even mantissa (1.0) wins;
    # 1+3*2^-8 ties between 1+2^-7 and 1+2^-6: even (1+2^-6) wins
    assert out[0] == 1.0 and out[1] == 1.0 and out[2] == np.float32(1 + 2 ** -6)
    assert out[3] == 1.0 and out[4] == -2.5
    assert abs(out[5] - 3.0e-3) <= 2 ** -8 * 3.0e-3   # unit roundoff of an 8-bit significand
    # decode is exact and round trip of representable values is the identity
    b = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(I.f32_to_bf16_bits(I.bf16_bits_to_f32(b)), b)


def test_chunked_draw_equals_single_draw(monkeypatch):
    a = I.make_inputs(2, 3, 8, 8, 1, dtype="f32", seed=5)
    monkeypatch.setattr(I, "_CHUNK", 7)
    b = I.make_inputs(2, 3, 8, 8, 1, dtype="f32", seed=5)
    for name in ("x", "dy", "w_base", "w_lvl", "scale"):
        assert np.array_equal(getattr(a, name), getattr(b, name))


def test_recipe_order_and_ranges():
    inp = I.make_inputs(2, 4, 16, 16, 2, kb=7, k=5, dtype="bf16", seed=0)
    assert inp.x.dtype == np.uint16 and inp.x.shape == (2, 4, 16, 16)
    assert inp.w_base.shape == (4, 7, 7) and inp.w_lvl.shape == (2, 4, 4, 5, 5)
    assert inp.scale.min() >= 0.5 and inp.scale.max() <= 1.5
    rng = np.random.default_rng(0)
    x = (1.0 * rng.standard_normal(2 * 4 * 16 * 16)).astype(np.float32)
    assert np.array_equal(I.f32_to_bf16_bits(x).reshape(inp.x.shape), inp.x)
