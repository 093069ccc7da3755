"""Pins of the oracle's dense linear: a hand-worked example, exact rational
brute force with the float64 error bound, and closed-form special cases."""
from fractions import Fraction

import numpy as np

from conftest import golden_dict
from fp4_block_scaled_route_amd import synth
from oracle import codec, linear, quant


def _golden_linear():
    g = golden_dict("linear_example.txt")
    w = np.array([[int(b, 16) for b in g["w_row0"]], [int(b, 16) for b in g["w_row1"]]], np.uint8)
    sf = np.array([[int(g["sf"][0], 16)], [int(g["sf"][1], 16)]], np.uint8)
    x = np.array([[float(v) for v in g["x_row0"]], [float(v) for v in g["x_row1"]]])
    y = np.array([[float(v) for v in g["y_row0"]], [float(v) for v in g["y_row1"]]])
    return x, w, sf, float(g["ws2"][0]), y


def test_hand_worked_linear():
    x, w, sf, ws2, y = _golden_linear()
    assert np.array_equal(linear.linear_bf16(x, w, sf, ws2), y)


def _exact_value_table():
    e2m1 = {}
    for c in range(16):
        s = -1 if c & 8 else 1
        e, m = (c >> 1) & 3, c & 1
        e2m1[c] = s * (Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2)))
    return e2m1


def _exact_e4m3(b):
    e, m = (b >> 3) & 15, b & 7
    return Fraction(m, 8) * Fraction(1, 64) if e == 0 else Fraction(2) ** (e - 7) * (1 + Fraction(m, 8))


def test_rational_brute_force_cfg1_within_float64_bound():
    """Single NVFP4 linear, seed 0: x [8,256], W [128,256], ws2 = 0.002.
    Every input is a dyadic rational, so y is computed exactly with Fractions;
    the float64 oracle must lie within gamma_K * sum|x w| (Higham, Accuracy and
    Stability of Numerical Algorithms, 2nd ed., section 3.1)."""
    li = synth.make_linear(8, 128, 256, seed=0)
    x = synth.bf16_to_float64(li.x)
    y = linear.linear_bf16(x, li.w, li.w_sf, li.ws2)
    tab = _exact_value_table()
    codes = codec.unpack_fp4(li.w)
    ws2 = Fraction(li.ws2)
    u = 2.0 ** -53
    gamma = 256 * u / (1 - 256 * u)
    for n in range(0, 128, 9):
        wn = [tab[int(codes[n, k])] * _exact_e4m3(int(li.w_sf[n, k // 16])) * ws2 for k in range(256)]
        for m in range(8):
            xm = [Fraction(float(v)) for v in x[m]]
            exact = sum(a * b for a, b in zip(xm, wn))
            absum = float(sum(abs(a * b) for a, b in zip(xm, wn)))
            assert abs(y[m, n] - float(exact)) <= gamma * absum + 1e-300


def test_one_hot_selects_a_dequantized_column():
    li = synth.make_linear(1, 32, 64, seed=5)
    wd = codec.dequant_nvfp4(li.w, li.w_sf, li.ws2)
    for k in (0, 1, 17, 63):
        x = np.zeros((1, 64))
        x[0, k] = 1.0
        assert np.array_equal(linear.linear_bf16(x, li.w, li.w_sf, li.ws2)[0], wd[:, k])


def test_scaling_and_zero_ws2():
    li = synth.make_linear(4, 32, 64, seed=6)
    x = synth.bf16_to_float64(li.x)
    y = linear.linear_bf16(x, li.w, li.w_sf, li.ws2)
    assert np.array_equal(linear.linear_bf16(x * 8.0, li.w, li.w_sf, li.ws2), y * 8.0)
    assert not linear.linear_bf16(x, li.w, li.w_sf, 0.0).any()


def test_nvfp4_activations_equal_linear_on_dequantized_x():
    li = synth.make_linear(4, 16, 64, seed=7)
    xp, xs, gs = quant.quantize_nvfp4(li.x.float().numpy())
    y4 = linear.linear_nvfp4(xp, xs, gs, li.w, li.w_sf, li.ws2)
    xd = quant.dequantize_nvfp4(xp, xs, gs)
    assert np.allclose(y4, linear.linear_bf16(xd, li.w, li.w_sf, li.ws2), rtol=1e-15, atol=0)


def test_layout_n_major_output_width():
    """Page "commit efe63ca", note on the N-major checkpoint layout: weights are
    [N, K/2]; a q_a-shaped weight [1536, 7168] must give 1536 outputs (a K/N swap
    gave 3584)."""
    w = np.zeros((1536, 7168 // 2), np.uint8)
    sf = np.zeros((1536, 7168 // 16), np.uint8)
    y = linear.linear_bf16(np.zeros((1, 7168)), w, sf, 1.0)
    assert y.shape == (1, 1536)
