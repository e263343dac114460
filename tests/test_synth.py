"""Host-side checks of the seeded input generator (no convolution arithmetic)."""
import numpy as np

from cnn_convolution_forward_amd import synth


def test_bf16_rounding_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -1.5, 1.0 + 2 ** -8 + 2 ** -20],
                 np.float32)
    bits = synth.f32_to_bf16_bits(f)
    back = synth.bf16_bits_to_f32(bits)
    # 1+2^-8 is a tie between 1 and 1+2^-7: even mantissa (1.0) wins;
    # 1+3*2^-8 ties between 1+2^-7 and 1+2^-6: the even one is 1+2^-6.
    np.testing.assert_array_equal(back, np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -1.5, 1.0 + 2 ** -7],
                                                 np.float32))


def test_workload_shapes():
    W = synth.WORKLOADS
    assert W["tiny_f32"].y_shape == (2, 4, 5, 6)
    assert W["stem_bf16"].y_shape == (32, 64, 112, 112)
    assert W["conv3x3_bf16"].y_shape == (64, 128, 56, 56)
    assert W["conv1x1_bf16"].y_shape == (32, 1024, 28, 28)
    assert W["conv3d_bf16"].y_shape == (8, 64, 16, 64, 64)
    assert W["conv3x3_bf16"].flops() == 2 * 64 * 128 * 56 * 56 * 128 * 9


def test_flop_formula_against_page_examples():
    # 2*8*128*32*32*64*9 ~ 1.2e9 (3x3) and 2*8*32*32*64*128 ~ 1.34e8 (pointwise)
    # [PyTorch tensor products and conv2d/conv3d dimension semantics, 3.3]
    wl3 = synth.Workload("x", 2, 8, 64, (32, 32), 128, 3, 1, 1, "bf16", "normal", 0)
    wl1 = synth.Workload("x", 2, 8, 64, (32, 32), 128, 1, 1, 0, "bf16", "normal", 0)
    assert abs(wl3.flops() / 1.2e9 - 1) < 0.01
    assert abs(wl1.flops() / 1.34e8 - 1) < 0.01


def test_generator_is_seeded_and_in_range():
    wl = synth.WORKLOADS["tiny_f32"]
    a, b = synth.make_inputs(wl), synth.make_inputs(wl)
    np.testing.assert_array_equal(a.x, b.x)
    assert a.x.dtype == np.float32 and np.all(np.abs(a.x) <= 1)
    wl = synth.workload("conv3x3_bf16", N=2)
    t = synth.make_inputs(wl)
    assert t.x.dtype == np.uint16 and t.x.shape == (2, 128, 56, 56)
    xf = synth.bf16_bits_to_f32(t.x)
    assert np.all(np.isfinite(xf))
    ti = synth.make_inputs(wl, integer=True)
    xi = synth.bf16_bits_to_f32(ti.x)
    assert set(np.unique(xi)) <= {-2, -1, 0, 1, 2}
    assert set(np.unique(ti.b)) <= set(range(-3, 4))
