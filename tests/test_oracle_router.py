"""Pins of the router oracle (oracle/router.py) against the page's rule,
hand-worked examples, library casts and exact arithmetic."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import codec, router


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(200_000).astype(np.float32),
                        (rng.standard_normal(20_000) * 1e30).astype(np.float32),
                        (rng.standard_normal(20_000) * 1e-30).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0], dtype=np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(router.bf16_round(v), ref)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: the even pattern is 1
    assert router.bf16_round(np.float32(1 + 2 ** -8)) == 1.0
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert router.bf16_round(np.float32(1 + 3 * 2 ** -8)) == 1 + 2 ** -6


def test_roundtrip_hand_worked_row():
    rows = read_golden("router_roundtrip_example.txt")
    w = np.array([float(r[0]) for r in rows], dtype=np.float32)
    b, scale, wr = router.router_weight_roundtrip(w[None, :])
    assert scale == np.float32(2.0 ** -7)
    assert [f"{x:02x}" for x in b[0]] == [r[1] for r in rows]
    assert np.array_equal(wr[0], np.array([float(r[2]) for r in rows]))


def test_fp8_quantize_matches_torch_float8_cast():
    rng = np.random.default_rng(5)
    w = torch.from_numpy(rng.standard_normal((64, 512)).astype(np.float32) * 0.02).to(torch.bfloat16)
    wf = w.float().numpy()
    scale = router.fp8_scale(wf)
    assert scale == np.float32(np.float32(np.abs(wf).max()) / np.float32(448.0))
    q = (wf / scale).astype(np.float32)
    assert np.abs(q).max() <= 448.0 * (1 + 2 ** -23)
    ref = torch.from_numpy(np.clip(q, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = router.fp8_quantize(wf, scale)
    # +-0 are the same value
    same = (got == ref) | (((got & 0x7F) == 0) & ((ref & 0x7F) == 0))
    assert same.all()
    # the largest magnitude maps to 448 exactly
    i = np.unravel_index(np.argmax(np.abs(wf)), wf.shape)
    assert got[i] & 0x7F == 0x7E


def test_fp8_dequant_is_bf16_of_fp32_product():
    scale = np.float32(0.0123)
    b = np.arange(256, dtype=np.uint8)
    b = b[(b & 0x7F) != 0x7F]                      # no NaN bytes
    vals = codec.E4M3_VALUES[b].astype(np.float32) * scale
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(router.fp8_dequant_bf16(b, scale), ref)


def test_roundtrip_is_idempotent_and_bounded():
    rng = np.random.default_rng(7)
    w = torch.from_numpy(rng.standard_normal((48, 256)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    _, scale, wr = router.router_weight_roundtrip(w)
    # relative error of E4M3 (2^-4) plus the bf16 rounding (2^-8), and the
    # absolute step of the smallest subnormal code
    err = np.abs(wr - w)
    assert np.all(err <= np.abs(w) * (2 ** -4 + 2 ** -8) + scale * 2.0 ** -9 + 1e-30)
    # values already on the grid come back unchanged when the scale is kept
    b2 = router.fp8_quantize(wr.astype(np.float32), scale)
    assert np.array_equal(router.fp8_dequant_bf16(b2, scale), wr)


def test_zero_weight_gives_zero():
    b, scale, wr = router.router_weight_roundtrip(np.zeros((3, 16), dtype=np.float32))
    assert scale == 0 and not b.any() and not wr.any()


def test_topk_hand_worked():
    for k, lg, ids, w in read_golden("router_topk_example.txt"):
        logits = np.array([[float(v) for v in lg.split(",")]])
        got_ids, got_w = router.topk_softmax(logits, int(k))
        assert got_ids[0].tolist() == [int(v) for v in ids.split(",")]
        assert np.allclose(got_w[0], [float(v) for v in w.split(",")], rtol=0, atol=1e-12)


def test_topk_against_brute_force_and_invariants():
    rng = np.random.default_rng(11)
    logits = rng.integers(-3, 4, size=(200, 24)).astype(np.float64)   # many ties
    ids, w = router.topk_softmax(logits, 5)
    for t in range(logits.shape[0]):
        ranked = sorted(range(24), key=lambda e: (-logits[t, e], e))[:5]
        assert ids[t].tolist() == ranked
        z = np.exp(logits[t, ranked] - logits[t, ranked[0]])
        assert np.allclose(w[t], z / z.sum(), rtol=0, atol=1e-15)
    assert np.allclose(w.sum(1), 1.0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 1e-15)       # weights ordered like the logits


def test_logits_exact_against_rational_brute_force():
    rng = np.random.default_rng(13)
    x = torch.from_numpy(rng.standard_normal((3, 40)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    w = torch.from_numpy(rng.standard_normal((6, 40)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    _, _, wr = router.router_weight_roundtrip(w)
    logits, ids, wts = router.route(x, wr, 2)
    for t in range(3):
        for e in range(6):
            exact = sum(Fraction(float(x[t, k])) * Fraction(float(wr[e, k])) for k in range(40))
            # float64 sum of 40 exact products: within 40 ulps of the largest partial sum
            assert abs(Fraction(float(logits[t, e])) - exact) <= Fraction(40 * 2.0 ** -52) * sum(
                abs(Fraction(float(x[t, k])) * Fraction(float(wr[e, k]))) for k in range(40))


@pytest.mark.parametrize("mistake", ["scale_inverted", "ties_high", "softmax_all", "no_bf16"])
def test_planted_mistakes_fail_a_pin(mistake):
    rows = read_golden("router_roundtrip_example.txt")
    w = np.array([float(r[0]) for r in rows], dtype=np.float32)[None, :]
    expect_wr = np.array([float(r[2]) for r in rows])
    topk_rows = read_golden("router_topk_example.txt")
    if mistake == "scale_inverted":
        scale = np.float32(448.0 / np.abs(w).max())
        wr = router.fp8_dequant_bf16(router.fp8_quantize(w, scale), scale)
        assert not np.array_equal(wr[0], expect_wr)
    elif mistake == "ties_high":
        k, lg, ids, _ = topk_rows[0]
        logits = np.array([float(v) for v in lg.split(",")])
        got = sorted(range(len(logits)), key=lambda e: (-logits[e], -e))[: int(k)]
        assert got != [int(v) for v in ids.split(",")]
    elif mistake == "softmax_all":
        k, lg, _, wts = topk_rows[2]
        logits = np.array([float(v) for v in lg.split(",")])
        z = np.exp(logits - logits.max())
        full = z / z.sum()
        got = np.sort(full)[::-1][: int(k)]
        assert not np.allclose(got, [float(v) for v in wts.split(",")], atol=1e-6)
    else:  # dequant kept in fp32, not rounded to bf16
        scale = np.float32(0.0123)
        b = np.array([0x35, 0x4B, 0x5E], dtype=np.uint8)
        wr32 = codec.E4M3_VALUES[b].astype(np.float32) * scale
        assert not np.array_equal(wr32.astype(np.float64), router.fp8_dequant_bf16(b, scale))
