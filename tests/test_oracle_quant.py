"""Pins of the oracle's activation quantizer: the global-scale closed form,
a hand-worked example, idempotence, and the pages' round-trip statistic."""
import numpy as np

from conftest import golden_dict
from oracle import codec, quant


def test_global_scale_closed_form():
    # gs = amax / (6 * 448): page "commit 4c6464e - vllm", note on the activation global scale
    for amax, gs in [(2688.0, 1.0), (336.0, 0.125), (6.0 * 448.0 * 2.0 ** -20, 2.0 ** -20), (0.0, 0.0)]:
        x = np.zeros((1, 16), np.float32)
        x[0, 3] = -amax
        assert quant.global_scale(x) == np.float32(gs)


def test_hand_worked_example():
    g = golden_dict("quantize_example.txt")
    x = np.array([[float(v) for v in g["x"]]], np.float32)
    packed, sb, gs = quant.quantize_nvfp4(x)
    assert gs == np.float32(float(g["gs"][0]))
    assert [int(b) for b in sb[0]] == [int(b, 16) for b in g["scale_bytes"]]
    assert [int(b) for b in packed[0]] == [int(b, 16) for b in g["packed"]]
    deq = quant.dequantize_nvfp4(packed, sb, gs)
    assert np.array_equal(deq[0], np.array([float(v) for v in g["dequant"]]))


def test_zero_tensor_gives_zero_codes_and_scales():
    packed, sb, gs = quant.quantize_nvfp4(np.zeros((3, 32), np.float32))
    assert gs == 0 and not packed.any() and not sb.any()


def test_codes_within_range_and_scales_within_448():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((16, 512)) * np.exp(rng.uniform(-2, 2, (16, 1)))).astype(np.float32)
    packed, sb, gs = quant.quantize_nvfp4(x)
    assert np.all(codec.E4M3_VALUES[sb] <= 448)
    deq = quant.dequantize_nvfp4(packed, sb, gs)
    # each element is within half a code step (<= 1 at magnitude 4..6) times its block scale
    s = codec.block_scales(sb, 512) * float(gs)
    err = np.abs(deq - x.astype(np.float64))
    assert np.all(err <= 1.0 * s + 1e-30)


def test_idempotent():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    p1, s1, gs = quant.quantize_nvfp4(x)
    d1 = quant.dequantize_nvfp4(p1, s1, gs).astype(np.float32)
    p2, s2, gs2 = quant.quantize_nvfp4(d1, gs=gs)
    assert np.array_equal(s1, s2)
    assert np.array_equal(codec.E2M1_VALUES[codec.unpack_fp4(p1)], codec.E2M1_VALUES[codec.unpack_fp4(p2)])


def test_round_trip_cosine_matches_pages():
    """Page "commit 1121cd7": NVFP4 round trip cos = 0.995 in isolation;
    page "commit 4c6464e": the standalone NVFP4 test passes at cos >= 0.994."""
    rng = np.random.Generator(np.random.PCG64(0))
    x = rng.standard_normal((64, 7168), dtype=np.float32)
    packed, sb, gs = quant.quantize_nvfp4(x)
    d = quant.dequantize_nvfp4(packed, sb, gs).ravel()
    xf = x.astype(np.float64).ravel()
    cos = xf @ d / np.linalg.norm(xf) / np.linalg.norm(d)
    assert 0.994 <= cos <= 0.997, cos


def test_supplied_gs_saturates():
    x = np.full((1, 16), 100.0, np.float32)
    packed, sb, gs = quant.quantize_nvfp4(x, gs=np.float32(0.01))   # 100/(6*.01) > 448
    assert sb[0, 0] == 0x7E
    assert np.all(codec.unpack_fp4(packed) == 7)
