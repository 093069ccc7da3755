"""Pins of the oracle's permutation, expert FFN and combine: hand-worked
examples, brute force and invariants."""
import numpy as np
import pytest

from conftest import golden_dict
from fp4_block_scaled_route_amd import synth
from oracle import codec, moe, quant


def test_permute_hand_worked():
    g = golden_dict("permute_example.txt")
    ids = np.array([int(v) for v in g["ids"]], np.int32).reshape(3, 2)
    off, perm, inv = moe.permute(ids, 3, has_shared=True)
    assert list(off) == [int(v) for v in g["offsets"]]
    assert list(perm) == [int(v) for v in g["perm"]]
    assert list(inv) == [int(v) for v in g["inv"]]


def _counting_sort_loop(ids, e):
    """Brute force: walk experts, then pairs in order (plain loops)."""
    flat = [int(v) for v in ids.reshape(-1)]
    perm, offsets = [], []
    for ex in range(e):
        offsets.append(len(perm))
        for f, v in enumerate(flat):
            if v == ex:
                perm.append(f)
    offsets.append(len(perm))
    return offsets, perm


@pytest.mark.parametrize("t,e,k,mode", [(64, 384, 8, "uniform"), (128, 384, 8, "zipf"), (7, 5, 3, "uniform"), (1, 16, 8, "zipf")])
def test_permute_brute_force_and_invariants(t, e, k, mode):
    ids, w = synth.route(t, e, k, seed=0, mode=mode)
    off, perm, inv = moe.permute(ids, e, has_shared=True)
    bo, bp = _counting_sort_loop(ids, e)
    assert list(off[:e + 1]) == bo and list(perm[:t * k]) == bp
    p = t * k
    assert off[0] == 0 and off[e] == p and off[e + 1] == p + t
    assert np.all(np.diff(off) >= 0)
    assert np.array_equal(np.diff(off[:e + 1]), np.bincount(ids.ravel(), minlength=e))
    assert sorted(perm) == list(range(p + t))
    assert np.array_equal(inv[perm], np.arange(p + t))
    flat = ids.ravel()
    for g in range(e):
        seg = perm[off[g]:off[g + 1]]
        assert np.all(flat[seg] == g) and np.all(np.diff(seg) > 0)


@pytest.mark.parametrize("mode", ["uniform", "zipf"])
def test_routing_invariants(mode):
    t, e, k = 256, 384, 8
    ids, w = synth.route(t, e, k, seed=1, mode=mode)
    assert ids.shape == (t, k) and ids.dtype == np.int32
    assert ids.min() >= 0 and ids.max() < e
    assert all(len(set(r)) == k for r in ids.tolist())          # k distinct experts per token
    assert np.all(w >= 0) and np.allclose(w.sum(1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 1e-7)                    # weights ordered like the logits


def test_zipf_routing_is_skewed():
    """Zipf(1.1) routing: selection frequency falls with the expert's Zipf rank
    (ranks are the seeded permutation the generator draws)."""
    seed, e = 2, 384
    ids, _ = synth.route(2048, e, 8, seed=seed, mode="zipf")
    counts = np.bincount(ids.ravel(), minlength=e)
    ranks = synth._rng(seed, synth._TAG_PERM).permutation(e) + 1
    assert counts[np.argmin(ranks)] == counts.max()             # rank 1 is the hottest
    assert counts.max() > 8 * counts.mean()
    c = np.corrcoef(np.log(ranks), np.log(counts + 1))[0, 1]
    assert c < -0.9, c


def _one_hot_swiglu_expert(h=16, i=16):
    w1c = np.zeros((2 * i, h), np.uint8)
    w1c[:i, 0] = 4            # code 4 = 2.0 (gate)
    w1c[i:, 0] = 2            # code 2 = 1.0 (up)
    w2c = np.zeros((h, i), np.uint8)
    np.fill_diagonal(w2c, 2)  # identity
    w1 = codec.pack_fp4(w1c)
    w2 = codec.pack_fp4(w2c)
    s1 = np.full((2 * i, h // 16), 0x38, np.uint8)
    s2 = np.full((h, i // 16), 0x38, np.uint8)
    return (w1, s1, 1.0, w2, s2, 1.0)


def test_swiglu_hand_worked():
    g = golden_dict("swiglu_example.txt")
    ex = _one_hot_swiglu_expert()
    x = np.zeros((1, 16))
    x[0, 0] = 1.0
    y = moe.moe_forward(x, np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32),
                        lambda e: ex, None)
    assert np.allclose(y[0], float(g["y_all"][0]), rtol=1e-15, atol=0)


def _small_moe(seed=0, t=6, h=256, i=256, e=5, k=2, shared=True):
    return synth.make_moe(t, h, i, e, k, seed=seed, shared=shared, threads=2)


def test_identical_experts_reduce_to_twice_one_ffn():
    mi = _small_moe()
    x = synth.bf16_to_float64(mi.x)
    ex0 = mi.experts.expert(0)
    y = moe.moe_forward(x, mi.topk_ids, mi.topk_w, lambda e: ex0, ex0)
    w1d = codec.dequant_nvfp4(ex0[0], ex0[1], ex0[2])
    w2d = codec.dequant_nvfp4(ex0[3], ex0[4], ex0[5])
    one = moe.expert_ffn(x, w1d, w2d)
    # routed weights sum to 1 (up to float32 rounding) and the shared expert adds 1
    want = (mi.topk_w.astype(np.float64).sum(1) + 1.0)[:, None] * one
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12 * np.abs(one).max())
    assert np.allclose(y, 2 * one, rtol=1e-6, atol=0)


def test_zeroing_a_weight_removes_exactly_that_pair():
    mi = _small_moe(seed=1, shared=False)
    x = synth.bf16_to_float64(mi.x)
    y = moe.moe_forward(x, mi.topk_ids, mi.topk_w, mi.experts.expert)
    w2 = mi.topk_w.copy()
    w2[3, 1] = 0
    y2 = moe.moe_forward(x, mi.topk_ids, w2, mi.experts.expert)
    e = int(mi.topk_ids[3, 1])
    ex = mi.experts.expert(e)
    o = moe.expert_ffn(x[3:4], codec.dequant_nvfp4(*ex[:3]), codec.dequant_nvfp4(*ex[3:]))
    assert np.allclose(y[3] - y2[3], mi.topk_w[3, 1] * o[0], rtol=1e-9, atol=1e-12)
    assert np.array_equal(np.delete(y, 3, 0), np.delete(y2, 3, 0))


def test_token_permutation_equivariance_and_subset():
    mi = _small_moe(seed=2)
    x = synth.bf16_to_float64(mi.x)
    y = moe.moe_forward(x, mi.topk_ids, mi.topk_w, mi.experts.expert, mi.shared.expert(0))
    p = np.random.default_rng(0).permutation(x.shape[0])
    yp = moe.moe_forward(x[p], mi.topk_ids[p], mi.topk_w[p], mi.experts.expert, mi.shared.expert(0))
    assert np.allclose(yp, y[p], rtol=1e-12, atol=0)
    ys = moe.moe_forward(x, mi.topk_ids, mi.topk_w, mi.experts.expert, mi.shared.expert(0), tokens=[4, 1])
    assert np.allclose(ys, y[[4, 1]], rtol=1e-12, atol=0)


def test_single_expert_equals_two_linears_and_silu():
    """E = 1, k = 1, w = 1: the MoE is W2 @ (silu(W1g x) * (W1u x))."""
    mi = _small_moe(seed=3, e=1, k=1, shared=False)
    x = synth.bf16_to_float64(mi.x)
    w1, s1, g1, w2, s2, g2 = mi.experts.expert(0)
    i = w1.shape[0] // 2
    from oracle import linear
    gate = linear.linear_bf16(x, w1[:i], s1[:i], g1)
    up = linear.linear_bf16(x, w1[i:], s1[i:], g1)
    h = gate / (1 + np.exp(-gate)) * up
    want = linear.linear_bf16(h, w2, s2, g2)
    got = moe.moe_forward(x, mi.topk_ids, np.ones_like(mi.topk_w), mi.experts.expert)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# fully-FP4 expert: h quantized with a2_gs before the down projection, and the
# warm-up calibration of a2_gs (tests/golden/fp4_hidden_example.txt)
# ---------------------------------------------------------------------------


def _tie_point_expert():
    """Case 2 of fp4_hidden_example.txt: g_i = 64 (silu exact), u_i = t_i / 64."""
    g = golden_dict("fp4_hidden_example.txt")
    w1c = np.zeros((32, 16), np.uint8)
    s1 = np.full((32, 1), 0x38, np.uint8)
    w1c[:16, 0] = 4                     # 2.0
    s1[:16, 0] = 0x60                   # 32
    w1c[16:, 0] = [int(v) for v in g["case2_up_codes"]]
    s1[16:, 0] = [int(v, 16) for v in g["case2_up_bytes"]]
    w2c = np.zeros((16, 16), np.uint8)
    np.fill_diagonal(w2c, 2)
    return (codec.pack_fp4(w1c), s1, 1.0, codec.pack_fp4(w2c), np.full((16, 1), 0x38, np.uint8), 1.0), g


def _e0():
    x = np.zeros((1, 16))
    x[0, 0] = 1.0
    return x


def _deq(ex):
    return codec.dequant_nvfp4(*ex[:3]), codec.dequant_nvfp4(*ex[3:])


def test_fp4_hidden_one_hot_hand_worked():
    g = golden_dict("fp4_hidden_example.txt")
    w1d, w2d = _deq(_one_hot_swiglu_expert())
    amax = moe.hidden_amax(_e0(), w1d)
    assert amax == float(g["case1_hidden_amax"][0])
    a2 = np.float32(np.float32(amax) / np.float32(2688.0))
    assert a2 == np.float32(float(g["case1_a2_gs"][0]))
    y = moe.expert_ffn(_e0(), w1d, w2d, a2_gs=a2)
    assert np.array_equal(y[0], np.full(16, float(g["case1_y_all"][0])))
    # the same through the MoE layer (E = 1, k = 1, w = 1)
    ym = moe.moe_forward(_e0(), np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32),
                         lambda e: _one_hot_swiglu_expert(), None, a2_gs=a2)
    assert np.array_equal(ym[0], y[0])


def test_fp4_hidden_tie_points_hand_worked():
    ex, g = _tie_point_expert()
    w1d, w2d = _deq(ex)
    want_h = np.array([float(v) for v in g["case2_h"]])
    # unquantized h: W2 is the identity, so y = h = t exactly
    assert np.array_equal(moe.expert_ffn(_e0(), w1d, w2d)[0], want_h)
    assert moe.hidden_amax(_e0(), w1d) == float(g["case2_hidden_amax"][0])
    y = moe.expert_ffn(_e0(), w1d, w2d, a2_gs=np.float32(1.0))
    assert np.array_equal(y[0], np.array([float(v) for v in g["case2_y"]]))
    # the h quantization itself: one block, scale byte and tie-to-even codes
    hp, hs, _ = quant.quantize_nvfp4(want_h[None].astype(np.float32), gs=np.float32(1.0))
    assert hs[0, 0] == int(g["case2_scale_byte"][0], 16)
    assert list(codec.unpack_fp4(hp)[0]) == [int(v) for v in g["case2_codes"]]
    # two tokens routed to the tie-point expert and the one-hot one, with weights
    x = np.vstack([_e0(), _e0()])
    ids = np.array([[0, 1], [1, 0]], np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.5]], np.float32)
    experts = {0: ex, 1: _one_hot_swiglu_expert()}
    ym = moe.moe_forward(x, ids, w, lambda e: experts[e], None, a2_gs=np.float32(1.0))
    y1 = moe.expert_ffn(_e0(), *_deq(experts[1]), a2_gs=np.float32(1.0))[0]
    assert np.array_equal(ym[0], 0.75 * y[0] + 0.25 * y1)
    assert np.array_equal(ym[1], 0.5 * y1 + 0.5 * y[0])
