"""Pins of the fused RMSNorm + NVFP4 quantization oracle (oracle/rmsnorm.py):
hand-worked rows, the closed form within one bf16 rounding, exact
power-of-two invariance, the bf16 rounding against torch's cast, the
composition with the (separately pinned) quantizer, and planted mistakes."""
import numpy as np
import pytest
import torch

from conftest import golden_dict
from fp4_block_scaled_route_amd import synth
from oracle import quant, rmsnorm


def _rows(tag):
    g = golden_dict("rmsnorm_example.txt")
    return [np.array([float(v) for v in g[f"{n}{tag}"]], dtype=np.float32) for n in "xwy"]


@pytest.mark.parametrize("tag", ["a", "b", "c"])
def test_hand_worked_rows(tag):
    x, w, y = _rows(tag)
    assert np.array_equal(rmsnorm.rmsnorm_bf16(x[None, :], w, 0.0)[0], y)


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(100_000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    assert np.array_equal(rmsnorm.bf16_round(v), ref)


def test_closed_form_within_one_bf16_rounding():
    x = synth.bf16_normal((37, 1536), 3).float().numpy()
    w = synth.bf16_normal((1536,), 4).float().numpy()
    eps = 1e-6
    y = rmsnorm.rmsnorm_bf16(x, w, eps).astype(np.float64)
    x64 = x.astype(np.float64)
    exact = x64 * w[None, :] / np.sqrt((x64 ** 2).mean(axis=1, keepdims=True) + float(np.float32(eps)))
    # bf16 rounding (unit roundoff 2^-8) plus the float32 roundings
    assert np.all(np.abs(y - exact) <= np.abs(exact) * (2 ** -8 + 2 ** -21) + 1e-30)


def test_power_of_two_scaling_is_exact():
    x = synth.bf16_normal((8, 512), 5).float().numpy()
    w = synth.bf16_normal((512,), 6).float().numpy()
    y = rmsnorm.rmsnorm_bf16(x, w, 0.0)
    for p in (-20, -3, 5, 30):
        assert np.array_equal(rmsnorm.rmsnorm_bf16(x * np.float32(2.0 ** p), w, 0.0), y)


def test_fused_equals_quantizer_on_the_bf16_output():
    x = synth.bf16_normal((16, 256), 7).float().numpy()
    w = synth.bf16_normal((256,), 8).float().numpy()
    y, p, s, g = rmsnorm.rmsnorm_quantize(x, w, 1e-6)
    p2, s2, g2 = quant.quantize_nvfp4(y)
    assert g == g2 and np.array_equal(p, p2) and np.array_equal(s, s2)


@pytest.mark.parametrize("mistake", ["sum_not_mean", "eps_outside_root", "no_weight", "no_bf16_before_quant"])
def test_planted_mistakes_fail_a_pin(mistake):
    if mistake == "sum_not_mean":
        x, w, y = _rows("a")
        r = np.float32(1.0 / np.sqrt(np.sum(x.astype(np.float64) ** 2)))
        assert not np.array_equal(rmsnorm.bf16_round(x * r * w), y)
    elif mistake == "eps_outside_root":
        x = synth.bf16_normal((4, 64), 9).float().numpy()
        w = np.ones(64, np.float32)
        eps = 0.25
        good = rmsnorm.rmsnorm_bf16(x, w, eps)
        r = (1.0 / (np.sqrt((x.astype(np.float64) ** 2).mean(axis=1)) + eps)).astype(np.float32)
        assert not np.array_equal(rmsnorm.bf16_round(x * r[:, None]), good)
    elif mistake == "no_weight":
        x, w, y = _rows("b")
        assert not np.array_equal(rmsnorm.rmsnorm_bf16(x[None, :], np.ones(16, np.float32), 0.0)[0], y)
    else:   # quantizing the float32 products instead of the bf16 output changes codes
        x = synth.bf16_normal((64, 512), 10).float().numpy()
        w = synth.bf16_normal((512,), 11).float().numpy()
        _, p, s, _ = rmsnorm.rmsnorm_quantize(x, w, 1e-6)
        r = rmsnorm.rms_scale(x, 1e-6)
        y32 = ((x * r[:, None]).astype(np.float32) * w[None, :]).astype(np.float32)
        p32, s32, _ = quant.quantize_nvfp4(y32)
        assert not (np.array_equal(p, p32) and np.array_equal(s, s32))
