"""Pins of the grouped-linear oracle (oracle/grouped_linear.py): reduction to
the dense linear per group, exact rational brute force, group permutation,
the NVFP4-activation identity, and planted mistakes that must fail a pin."""
from fractions import Fraction

import numpy as np
import pytest

from fp4_block_scaled_route_amd import synth
from oracle import codec, grouped_linear, linear, quant


def _exact_e2m1(c):
    s = -1 if c & 8 else 1
    e, m = (c >> 1) & 3, c & 1
    return s * (Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2)))


def _exact_e4m3(b):
    e, m = (b >> 3) & 15, b & 7
    return Fraction(m, 8) * Fraction(1, 64) if e == 0 else Fraction(2) ** (e - 7) * (1 + Fraction(m, 8))


def test_each_group_is_the_dense_linear_of_its_slice():
    gi = synth.make_grouped_linear(5, 8, 24, 64, seed=1)
    x = synth.bf16_to_float64(gi.x)
    y = grouped_linear.grouped_linear_bf16(x, gi.w, gi.w_sf, gi.ws2)
    assert y.shape == (5, 8, 24)
    for g in range(8):
        ref = linear.linear_bf16(x[:, g, :], gi.w[g], gi.w_sf[g], float(gi.ws2[g]))
        assert np.allclose(y[:, g, :], ref, rtol=1e-13, atol=1e-300)


def test_rational_brute_force_within_float64_bound():
    """Every input is a dyadic rational: y[t, g, n] is computed exactly and the
    float64 oracle must lie within gamma_K * sum |x w| (Higham, section 3.1)."""
    gi = synth.make_grouped_linear(2, 3, 4, 32, seed=2)
    x = synth.bf16_to_float64(gi.x)
    y = grouped_linear.grouped_linear_bf16(x, gi.w, gi.w_sf, gi.ws2)
    u = 2.0 ** -53
    gamma = 32 * u / (1 - 32 * u)
    for g in range(3):
        codes = codec.unpack_fp4(gi.w[g])
        ws2 = Fraction(float(gi.ws2[g]))
        for n in range(4):
            wn = [_exact_e2m1(int(codes[n, k])) * _exact_e4m3(int(gi.w_sf[g, n, k // 16])) * ws2 for k in range(32)]
            for t in range(2):
                terms = [Fraction(float(v)) * w for v, w in zip(x[t, g], wn)]
                exact = sum(terms)
                assert abs(y[t, g, n] - float(exact)) <= gamma * float(sum(abs(v) for v in terms)) + 1e-300


def test_permuting_groups_permutes_outputs():
    gi = synth.make_grouped_linear(3, 8, 16, 64, seed=3)
    x = synth.bf16_to_float64(gi.x)
    y = grouped_linear.grouped_linear_bf16(x, gi.w, gi.w_sf, gi.ws2)
    p = np.array([3, 0, 7, 1, 6, 2, 5, 4])
    yp = grouped_linear.grouped_linear_bf16(x[:, p, :], gi.w[p], gi.w_sf[p], gi.ws2[p])
    assert np.array_equal(yp, y[:, p, :])


def test_nvfp4_activations_equal_bf16_path_on_dequantized_x():
    gi = synth.make_grouped_linear(4, 2, 16, 64, seed=4)
    xf = gi.x.float().numpy().reshape(8, 64)
    packed, sbytes, gs = quant.quantize_nvfp4(xf)
    y4 = grouped_linear.grouped_linear_nvfp4(packed.reshape(4, 2, 32), sbytes.reshape(4, 2, 4), gs,
                                             gi.w, gi.w_sf, gi.ws2)
    xd = quant.dequantize_nvfp4(packed, sbytes, gs).reshape(4, 2, 64)
    assert np.allclose(y4, grouped_linear.grouped_linear_bf16(xd, gi.w, gi.w_sf, gi.ws2), rtol=1e-13, atol=1e-300)


@pytest.mark.parametrize("mistake", ["shifted_group", "shared_ws2", "transposed_tg"])
def test_planted_mistakes_fail_the_per_group_pin(mistake):
    gi = synth.make_grouped_linear(3, 4, 8, 32, seed=5)
    x = synth.bf16_to_float64(gi.x)
    ref = np.stack([linear.linear_bf16(x[:, g, :], gi.w[g], gi.w_sf[g], float(gi.ws2[g])) for g in range(4)], axis=1)
    if mistake == "shifted_group":          # group g multiplied by the weight of group g+1
        y = grouped_linear.grouped_linear_bf16(x, np.roll(gi.w, 1, axis=0), np.roll(gi.w_sf, 1, axis=0), gi.ws2)
    elif mistake == "shared_ws2":           # one weight_scale_2 for every group
        y = grouped_linear.grouped_linear_bf16(x, gi.w, gi.w_sf, np.full(4, gi.ws2[0]))
    else:                                   # the [T, G, K] input read as [G, T, K]
        xt = x.reshape(4, 3, 32).transpose(1, 0, 2)
        y = grouped_linear.grouped_linear_bf16(xt, gi.w, gi.w_sf, gi.ws2)
    assert not np.allclose(y, ref, rtol=1e-6)
