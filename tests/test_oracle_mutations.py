"""Planted mistakes in the oracle must be caught by its pins.

Each case patches one oracle function (in memory, on the CPU) with a
plausible mistake, most of them bugs the pages record, and checks that at
least one pin test fails."""
import numpy as np
import pytest

import test_oracle_codec as tc
import test_oracle_linear as tl
import test_oracle_moe as tm
import test_oracle_quant as tq
from oracle import codec, moe, quant


def _must_fail(*pins):
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, "planted mistake went unnoticed"


def test_nibble_order_swapped(monkeypatch):
    orig = codec.unpack_fp4

    def swapped(p):
        c = orig(p)
        out = c.copy()
        out[..., 0::2], out[..., 1::2] = c[..., 1::2], c[..., 0::2]
        return out
    monkeypatch.setattr(codec, "unpack_fp4", swapped)
    _must_fail(tc.test_dequant_hand_worked_examples, tl.test_hand_worked_linear)


def test_weight_scale_2_dropped(monkeypatch):
    # page "commit efe63ca": weight_scale_2 dropped from the dequant
    orig = codec.dequant_nvfp4
    monkeypatch.setattr(codec, "dequant_nvfp4", lambda p, s, g: orig(p, s, 1.0))
    _must_fail(tc.test_dequant_hand_worked_examples, tl.test_hand_worked_linear)


def test_input_scale_folded_into_weights(monkeypatch):
    # page "commit 1121cd7" / "commit efe63ca": an activation scale folded into the weight dequant
    orig = codec.dequant_nvfp4
    monkeypatch.setattr(codec, "dequant_nvfp4", lambda p, s, g: orig(p, s, g * 2.5e-4))
    _must_fail(tl.test_hand_worked_linear)


def test_global_scale_inverted(monkeypatch):
    # page "commit 4c6464e": gs was wrongly inverted
    monkeypatch.setattr(quant, "global_scale",
                        lambda x: np.float32(quant.GS_DIVISOR / np.float32(np.max(np.abs(x))))
                        if np.max(np.abs(x)) else np.float32(0))
    _must_fail(tq.test_global_scale_closed_form)


def test_scales_transposed(monkeypatch):
    # page "commit efe63ca": scales read with K_sf and N swapped
    orig = codec.block_scales
    monkeypatch.setattr(codec, "block_scales",
                        lambda sf, k: orig(np.ascontiguousarray(np.asarray(sf).T).reshape(np.asarray(sf).shape), k))
    _must_fail(tl.test_rational_brute_force_cfg1_within_float64_bound)


def test_e2m1_ties_away_from_zero(monkeypatch):
    def away(v):
        v = np.asarray(v)
        mag = np.abs(v.astype(np.float64))
        vals = codec.E2M1_VALUES[:8]
        d = np.abs(mag[..., None] - vals)
        code = np.argmax(np.where(d == d.min(-1, keepdims=True), np.arange(8), -1), axis=-1)
        return (code | (np.signbit(v).astype(np.uint8) << 3)).astype(np.uint8)
    monkeypatch.setattr(codec, "e2m1_encode", away)
    _must_fail(tc.test_e2m1_rne_ties, tq.test_hand_worked_example)


def test_gate_and_up_swapped(monkeypatch):
    def swapped(a, w1d, w2d, a2_gs=None):
        i = w1d.shape[0] // 2
        return moe.__dict__["_orig_ffn"](a, np.concatenate([w1d[i:], w1d[:i]]), w2d, a2_gs)
    monkeypatch.setitem(moe.__dict__, "_orig_ffn", moe.expert_ffn)
    monkeypatch.setattr(moe, "expert_ffn", swapped)
    _must_fail(tm.test_swiglu_hand_worked)


def test_unstable_permutation(monkeypatch):
    orig = np.argsort

    def unstable(a, *args, **kw):
        kw["kind"] = "quicksort"
        r = orig(a, *args, **kw)
        # make ties come out reversed, the way an unstable sort may
        a = np.asarray(a)
        out = r.copy()
        i = 0
        while i < len(r):
            j = i
            while j < len(r) and a[r[j]] == a[r[i]]:
                j += 1
            out[i:j] = np.sort(r[i:j])[::-1]
            i = j
        return out
    monkeypatch.setattr(moe.np, "argsort", unstable)
    _must_fail(tm.test_permute_hand_worked)


def test_routing_weights_before_down_projection_not_distinguishable_is_caught(monkeypatch):
    # weights applied to the wrong pair (j reversed) must break the single-pair test
    orig = moe.moe_forward

    def wrong(x, ids, w, ew, sw=None, a2_gs=None, tokens=None):
        return orig(x, ids, np.asarray(w)[:, ::-1], ew, sw, a2_gs, tokens)
    monkeypatch.setattr(moe, "moe_forward", wrong)
    _must_fail(tm.test_zeroing_a_weight_removes_exactly_that_pair)


def _mutated_ffn(hidden):
    """expert_ffn with its h step replaced by ``hidden(h, a2_gs)``."""
    def ffn(a, w1d, w2d, a2_gs=None):
        i = w1d.shape[0] // 2
        h = moe.silu(a @ w1d[:i].T) * (a @ w1d[i:].T)
        if a2_gs is not None:
            h = hidden(h, a2_gs)
        return h @ w2d.T
    return ffn


_FP4_HIDDEN_PINS = (tm.test_fp4_hidden_one_hot_hand_worked, tm.test_fp4_hidden_tie_points_hand_worked)


def test_hidden_dequantized_with_doubled_scale(monkeypatch):
    # h dequantized with 2 * a2_gs (a global scale applied twice)
    def twice(h, gs):
        hp, hs, g = quant.quantize_nvfp4(h.astype(np.float32), gs=gs)
        return quant.dequantize_nvfp4(hp, hs, np.float32(2 * g))
    monkeypatch.setattr(moe, "expert_ffn", _mutated_ffn(twice))
    _must_fail(*_FP4_HIDDEN_PINS)


def test_hidden_not_quantized(monkeypatch):
    # a2_gs given but h passed to the down projection unquantized
    monkeypatch.setattr(moe, "expert_ffn", _mutated_ffn(lambda h, gs: h))
    _must_fail(*_FP4_HIDDEN_PINS)


def test_hidden_global_scale_inverted(monkeypatch):
    # page "commit 4c6464e": the global scale used inverted
    def inverted(h, gs):
        hp, hs, g = quant.quantize_nvfp4(h.astype(np.float32), gs=np.float32(1.0 / gs))
        return quant.dequantize_nvfp4(hp, hs, g)
    monkeypatch.setattr(moe, "expert_ffn", _mutated_ffn(inverted))
    _must_fail(tm.test_fp4_hidden_one_hot_hand_worked)


def test_hidden_amax_without_swiglu(monkeypatch):
    # calibration amax taken over the gate * up product instead of silu(gate) * up
    def amax(a, w1d):
        i = w1d.shape[0] // 2
        h = (a @ w1d[:i].T) * (a @ w1d[i:].T)
        return float(np.max(np.abs(h.astype(np.float32)))) if h.size else 0.0
    monkeypatch.setattr(moe, "hidden_amax", amax)
    _must_fail(tm.test_fp4_hidden_one_hot_hand_worked)
