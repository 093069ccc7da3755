"""CPU checks of the per-element error bound (tests/moe_bound.py) used by the
GPU parity tests: a numpy emulation of the GPU path's arithmetic (fp16
staging with per-row shifts, fp32 accumulation, fp32 SwiGLU, bf16 rows,
fp32 combine, bf16 output) stays inside the bound, and planted mistakes of
the kind the whole-tensor tolerance can miss fall outside it."""
import numpy as np
import pytest
import torch

from fp4_block_scaled_route_amd import synth
from moe_bound import reference_and_bound
from oracle import codec, quant

F32 = np.float32


def _bf16(v):
    return torch.from_numpy(np.ascontiguousarray(v, dtype=F32)).to(torch.bfloat16).float().numpy()


def _shift(rows):
    """Per-row power of two that puts the row maximum in [2^14, 2^15)."""
    m = np.abs(rows).max(axis=1)
    e = np.floor(np.log2(np.where(m > 0, m, 1.0)))
    return np.where(m > 0, 14 - e, 0).astype(np.int64)


def _raw(packed, sf):
    """E2M1 x E4M3 values (exact in fp32) without weight_scale_2."""
    return codec.dequant_nvfp4(packed, sf, 1.0).astype(F32)


def _emulate(mi, a2_gs=None, x_rows=None, w2_sf_override=None, slot_hook=None):
    """GPU arithmetic of one MoE layer, emulated on the CPU."""
    ex, t_all = mi.experts, mi.topk_ids.shape[0]
    x = synth.bf16_to_float64(mi.x) if x_rows is None else x_rows
    fp4_x = x_rows is not None
    sh = _shift(x)
    xs = x * np.exp2(sh)[:, None]
    a16 = xs.astype(F32) if fp4_x else xs.astype(np.float16).astype(F32)
    k = mi.topk_ids.shape[1]
    slots = {}

    def pair(t, w1, s1, g1, w2, s2, g2):
        i = w1.shape[0] // 2
        w1q, w2q = _raw(w1, s1), _raw(w2, s2)
        alpha1 = F32(g1) if not fp4_x else F32(F32(g1) * F32(1.0))
        acc = (a16[t:t + 1] @ w1q.T).astype(F32)
        gu = (np.ldexp(acc, -int(sh[t])) * alpha1).astype(F32)
        g, u = gu[:, :i], gu[:, i:]
        h = (g / (F32(1) + np.exp(-g)) * u).astype(F32)
        if a2_gs is None:
            s = _shift(h)
            h16 = (h * np.exp2(s)[:, None].astype(F32)).astype(np.float16).astype(F32)
            o = np.ldexp((h16 @ w2q.T).astype(F32), -int(s[0])) * F32(g2)
        else:
            hp, hs, _ = quant.quantize_nvfp4(h, gs=F32(a2_gs))
            hq = _raw(hp, hs)
            o = (hq @ w2q.T).astype(F32) * F32(F32(g2) * F32(a2_gs))
        return _bf16(o)[0]

    for t in range(t_all):
        for j in range(k):
            e = int(mi.topk_ids[t, j])
            w1, s1, g1, w2, s2, g2 = ex.expert(e)
            if w2_sf_override is not None and e in w2_sf_override:
                s2 = w2_sf_override[e]
            slots[(t, j)] = pair(t, w1, s1, g1, w2, s2, g2)
        if mi.shared is not None:
            slots[(t, -1)] = pair(t, *mi.shared.expert(0))
    if slot_hook is not None:
        slot_hook(slots)
    y = np.zeros((t_all, x.shape[1]), dtype=F32)
    for t in range(t_all):
        acc = np.zeros(x.shape[1], dtype=F32)
        for j in range(k):
            acc = (acc + F32(mi.topk_w[t, j]) * slots[(t, j)]).astype(F32)
        if (t, -1) in slots:
            acc = (acc + slots[(t, -1)]).astype(F32)
        y[t] = _bf16(acc)
    return y.astype(np.float64)


@pytest.fixture(scope="module")
def layer():
    mi = synth.make_moe(6, 512, 256, 5, 3, seed=3, shared=True, threads=2)
    x = synth.bf16_to_float64(mi.x)
    y_ref, bound, _ = reference_and_bound(x, mi.topk_ids, mi.topk_w, mi.experts, mi.shared, workers=2)
    return mi, y_ref, bound


def _ratio(y, y_ref, bound):
    return float(np.max(np.abs(y - y_ref) / bound))


def _normwise(y, y_ref):
    return float(np.abs(y - y_ref).max() / np.abs(y_ref).max())


def test_emulated_gpu_arithmetic_is_inside_the_bound(layer):
    mi, y_ref, bound = layer
    y = _emulate(mi)
    r = _ratio(y, y_ref, bound)
    assert r <= 1.0, r
    # the bound is an error bound, not a loose envelope: typical elements
    # are bounded at a few percent of their magnitude
    assert np.median(bound / np.abs(y_ref)) < 0.05


def test_doubled_scale_byte_breaks_the_bound(layer):
    mi, y_ref, bound = layer
    e = int(mi.topk_ids[2, 1])
    s2 = mi.experts.expert(e)[4].copy()
    s2[7, 3] = min(s2[7, 3] + 8, 0x7E)        # exponent + 1: that block's scale doubled
    y = _emulate(mi, w2_sf_override={e: s2})
    assert _ratio(y, y_ref, bound) > 1.0


def test_misindexed_row_breaks_the_bound(layer):
    mi, y_ref, bound = layer

    def swap(slots):
        slots[(1, 0)], slots[(4, 2)] = slots[(4, 2)].copy(), slots[(1, 0)].copy()
    assert _ratio(_emulate(mi, slot_hook=swap), y_ref, bound) > 1.0


def test_one_mantissa_step_of_one_scale_byte_breaks_the_bound(layer):
    """One block scale byte one mantissa step off (scale 1/8 to 1/16 larger):
    inside the whole-tensor tolerance (normwise 2e-2), outside the bound."""
    mi, y_ref, bound = layer
    e = int(mi.topk_ids[2, 1])
    s2 = mi.experts.expert(e)[4].copy()
    s2[7, 3] += 1
    y = _emulate(mi, w2_sf_override={e: s2})
    assert _normwise(y, y_ref) < 2e-2
    assert _ratio(y, y_ref, bound) > 1.0


def test_lowest_weight_row_dropped_breaks_the_bound(layer):
    """The output row of a token's lowest-weighted pair lost (as an indexing
    bug that never writes it would leave it)."""
    mi, y_ref, bound = layer
    t, j = 0, int(np.argmin(mi.topk_w[0]))

    def drop(slots):
        slots[(t, j)] = slots[(t, j)] * 0
    y = _emulate(mi, slot_hook=drop)
    assert _ratio(y, y_ref, bound) > 1.0


def test_fully_fp4_emulation_is_inside_the_bound():
    mi = synth.make_moe(6, 512, 256, 5, 3, seed=4, shared=False, threads=2)
    rq, rs, rgs = quant.quantize_nvfp4(mi.x.float().numpy())
    xa = quant.dequantize_nvfp4(rq, rs, rgs)
    from oracle import moe
    amax = 0.0
    for t in range(6):
        for j in range(3):
            ex = mi.experts.expert(int(mi.topk_ids[t, j]))
            amax = max(amax, moe.hidden_amax(xa[t:t + 1], codec.dequant_nvfp4(*ex[:3])))
    a2 = F32(F32(amax) / F32(2688.0))
    y_ref, bound, mb = reference_and_bound(xa, mi.topk_ids, mi.topk_w, mi.experts, None, a2_gs=a2,
                                           x_fp4=True, workers=2)
    y = _emulate(mi, a2_gs=a2, x_rows=xa)
    assert _ratio(y, y_ref, bound) <= 1.0

    def swap(slots):
        slots[(0, 0)], slots[(5, 1)] = slots[(5, 1)].copy(), slots[(0, 0)].copy()
    assert _ratio(_emulate(mi, a2_gs=a2, x_rows=xa, slot_hook=swap), y_ref, bound) > 1.0
