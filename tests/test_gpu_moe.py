"""GPU parity of nvfp4_moe_grouped against the oracle.

Every output element is checked twice: against the stated tolerance
(normwise max error 2e-2 of max|ref| and cosine 0.999) and against its own
error bound derived from the GPU path's arithmetic (tests/moe_bound.py).
Small shapes are compared in full.  The DeepSeek-V4-shaped configurations
(hidden 7168, intermediate 2048, 384 experts, top-8) run on the GPU at full
size in the launch configuration the benchmark times: the decode and prefill
batches are compared on every token, the 4096-token fully-FP4 batch on a
token set that routes to every one of the 384 experts.  The permutation
(segment offsets and sorted-row order) is compared bit for bit at every
size."""
import numpy as np
import pytest
import torch

from gpu_util import DeviceExperts, calibrate_a2, compare, covering_tokens, dev, f32, full_size_experts, say
from fp4_block_scaled_route_amd import ops, synth
from moe_bound import check_elementwise, reference_and_bound
from oracle import codec, moe, quant

pytestmark = pytest.mark.gpu


def _run(de, ids, w, x=None, shared=None, x_fp4=None, x_sf=None, a1_gs=None, a2_gs=None, a2_gs_out=None):
    t, k = ids.shape
    e = de.w1.shape[0]
    off = torch.empty(e + 2, dtype=torch.int32, device="cuda")
    perm = torch.empty(t * k + t, dtype=torch.int32, device="cuda")
    y = ops.moe_grouped(dev(ids), dev(w), **de.args(), x=x, x_fp4=x_fp4, x_sf=x_sf, a1_gs=a1_gs,
                        shared=shared.as_shared() if shared is not None else None,
                        a2_gs=a2_gs, a2_gs_out=a2_gs_out, offsets_out=off, perm_out=perm)
    torch.cuda.synchronize()
    return y, off.cpu().numpy(), perm.cpu().numpy()


def _check_perm(ids, e, has_shared, off, perm):
    ro, rp, _ = moe.permute(ids, e, has_shared)
    assert np.array_equal(off, ro), "segment offsets differ"
    n = ro[-1]
    assert np.array_equal(perm[:n], rp), "sorted-row order differs"


def _check(y_gpu, x_rows, ids, w, host, shared_host, tokens=None, a2_gs=None, x_fp4=False, what=""):
    """The oracle on ``tokens`` (default all) and both criteria: the stated
    tolerance and the per-element bound."""
    ref, bound, mb = reference_and_bound(x_rows, ids, w, host, shared_host, tokens=tokens, a2_gs=a2_gs,
                                         x_fp4=x_fp4, workers=16)
    g = y_gpu if tokens is None else y_gpu[torch.as_tensor(np.asarray(tokens), device=y_gpu.device)]
    g = g.float().cpu().numpy().astype(np.float64)
    compare(g, ref, what=what)
    check_elementwise(g, ref, bound, what=what)
    if a2_gs is not None:
        say(f"  {what}: {mb.flips} h elements within their error of an NVFP4 rounding boundary")


@pytest.mark.parametrize("t,h,i,e,k,routing,shared", [
    (37, 512, 256, 16, 4, "uniform", True),
    (64, 256, 512, 8, 2, "zipf", False),
    (1, 256, 256, 4, 4, "uniform", True),
    (300, 256, 256, 6, 3, "zipf", True),     # hot groups with > 128 rows: several passes
    (24, 256, 256, 16, 10, "uniform", True),  # top-10: the combine's loop for more than 8 pairs
])
def test_moe_small_bf16(t, h, i, e, k, routing, shared):
    say(f"moe bf16 T={t} H={h} I={i} E={e} k={k} {routing} shared={shared}")
    mi = synth.make_moe(t, h, i, e, k, seed=4, routing=routing, shared=shared, threads=4)
    de = DeviceExperts(mi.experts)
    ds = DeviceExperts(mi.shared) if shared else None
    y, off, perm = _run(de, mi.topk_ids, mi.topk_w, x=dev(mi.x), shared=ds)
    _check_perm(mi.topk_ids, e, shared, off, perm)
    _check(y, synth.bf16_to_float64(mi.x), mi.topk_ids, mi.topk_w, mi.experts, mi.shared, what="moe small")


def test_moe_identical_experts_invariant():
    """All experts (and the shared one) identical: y = (sum_j w + 1) * FFN(x)
    whatever the routing; checks weights and combine without indexing."""
    t, h, i, e, k = 20, 256, 256, 6, 3
    mi = synth.make_moe(t, h, i, e, k, seed=5, shared=True, threads=2)
    one = synth.make_experts(1, h, i, seed=9)
    same = synth.ExpertSet(*(np.repeat(a, e, axis=0) for a in
                             (one.w1, one.w1_sf, one.w1_ws2, one.w2, one.w2_sf, one.w2_ws2)))
    y, _, _ = _run(DeviceExperts(same), mi.topk_ids, mi.topk_w, x=dev(mi.x), shared=DeviceExperts(one))
    x = synth.bf16_to_float64(mi.x)
    ex = one.expert(0)
    f = moe.expert_ffn(x, codec.dequant_nvfp4(*ex[:3]), codec.dequant_nvfp4(*ex[3:]))
    ref = (mi.topk_w.astype(np.float64).sum(1) + 1.0)[:, None] * f
    compare(y, ref, what="identical experts")
    _check(y, x, mi.topk_ids, mi.topk_w, same, one, what="identical experts, oracle")


def test_moe_out_of_range_ids_contribute_nothing():
    t, h, i, e, k = 8, 256, 256, 4, 2
    mi = synth.make_moe(t, h, i, e, k, seed=6, shared=False, threads=2)
    ids = mi.topk_ids.copy()
    ids[2, 1] = e + 3
    ids[5, 0] = -1
    de = DeviceExperts(mi.experts)
    y, _, _ = _run(de, ids, mi.topk_w, x=dev(mi.x))
    w = mi.topk_w.copy()
    w[2, 1] = 0
    w[5, 0] = 0
    ids_ok = ids.copy()
    ids_ok[2, 1] = 0
    ids_ok[5, 0] = 0
    _check(y, synth.bf16_to_float64(mi.x), ids_ok, w, mi.experts, None, what="invalid ids")


def test_moe_small_fully_fp4_and_calibration():
    t, h, i, e, k = 40, 512, 512, 8, 4
    say("moe fully fp4 small")
    mi = synth.make_moe(t, h, i, e, k, seed=7, shared=True, threads=2)
    de, ds = DeviceExperts(mi.experts), DeviceExperts(mi.shared)
    # calibration call (h kept fp32): a2_gs_out = max|h| / 2688
    xq, xs, gs = ops.quantize_act(dev(mi.x))
    gs_out = f32(0)
    _run(de, mi.topk_ids, mi.topk_w, x_fp4=xq, x_sf=xs, a1_gs=gs, shared=ds, a2_gs_out=gs_out)
    rq, rs, rgs = quant.quantize_nvfp4(mi.x.float().numpy())
    xa = quant.dequantize_nvfp4(rq, rs, rgs)
    a2 = calibrate_a2(xa, mi.topk_ids, mi.experts, range(t), mi.shared)
    assert abs(gs_out.item() - a2) <= 1e-4 * a2, (gs_out.item(), a2)
    # fully FP4 call with the oracle's calibrated scale
    y, off, perm = _run(de, mi.topk_ids, mi.topk_w, x_fp4=xq, x_sf=xs, a1_gs=gs, shared=ds, a2_gs=f32(a2))
    _check_perm(mi.topk_ids, e, True, off, perm)
    _check(y, xa, mi.topk_ids, mi.topk_w, mi.experts, mi.shared, a2_gs=a2, x_fp4=True, what="fully fp4 small")


@pytest.mark.parametrize("t,h,i,e,k,seed", [
    (160, 1024, 1024, 24, 4, 11),   # K multiple of 1024: eight-wave kernel for both GEMMs
    (150, 512, 256, 20, 3, 12),     # four-wave large-batch configuration
    (160, 1280, 1024, 24, 4, 14),   # eight-wave down GEMM with a ragged last 512-row block (H = 1280)
])
def test_moe_large_batch_with_tiny_groups(t, h, i, e, k, seed):
    """More than 16 rows per group on average sends every group, including
    groups of 1-4 rows, to the LDS kernel in one launch; hot groups take
    several passes.  Zipf(1.6) routing gives both."""
    say(f"moe large batch with tiny groups T={t} H={h} I={i} E={e} k={k}")
    mi = synth.make_moe(t, h, i, e, k, seed=seed, routing="zipf", zipf_s=1.6, shared=True, threads=4)
    counts = np.bincount(mi.topk_ids.ravel(), minlength=e)
    assert (t * k + t) / (e + 1) > 16 and ((counts > 0) & (counts <= 4)).any() and counts.max() > 128
    de, ds = DeviceExperts(mi.experts), DeviceExperts(mi.shared)
    y, off, perm = _run(de, mi.topk_ids, mi.topk_w, x=dev(mi.x), shared=ds)
    _check_perm(mi.topk_ids, e, True, off, perm)
    _check(y, synth.bf16_to_float64(mi.x), mi.topk_ids, mi.topk_w, mi.experts, mi.shared,
           what="large batch, tiny groups")


def test_moe_fully_fp4_large_batch_with_tiny_groups():
    """The fully-FP4 path on the eight-wave kernel with groups of 1-4 rows and
    groups of more than one 112-row pass."""
    t, h, i, e, k = 192, 1024, 1024, 24, 4
    say("moe fully fp4 large batch with tiny groups")
    mi = synth.make_moe(t, h, i, e, k, seed=13, routing="zipf", zipf_s=1.6, shared=False, threads=4)
    counts = np.bincount(mi.topk_ids.ravel(), minlength=e)
    assert ((counts > 0) & (counts <= 4)).any() and counts.max() > 112
    de = DeviceExperts(mi.experts)
    xq, xs, gs = ops.quantize_act(dev(mi.x))
    rq, rs, rgs = quant.quantize_nvfp4(mi.x.float().numpy())
    xa = quant.dequantize_nvfp4(rq, rs, rgs)
    a2 = calibrate_a2(xa, mi.topk_ids, mi.experts, range(t))
    y, off, perm = _run(de, mi.topk_ids, mi.topk_w, x_fp4=xq, x_sf=xs, a1_gs=gs, a2_gs=f32(a2))
    _check_perm(mi.topk_ids, e, False, off, perm)
    _check(y, xa, mi.topk_ids, mi.topk_w, mi.experts, None, a2_gs=a2, x_fp4=True, what="fully fp4, tiny groups")


def test_moe_permutation_on_several_workgroups():
    """8800 pairs (more than 8191): the permutation runs on nine workgroups of
    consecutive 1024-pair ranges, the last one ragged; offsets and sorted-row
    order stay bit-exact, and so do they with ids out of range (those pairs
    take no row and contribute nothing)."""
    t, h, i, e, k = 1100, 256, 256, 64, 8
    say("moe permutation on several workgroups")
    mi = synth.make_moe(t, h, i, e, k, seed=21, routing="zipf", shared=True, threads=4)
    de, ds = DeviceExperts(mi.experts), DeviceExperts(mi.shared)
    y, off, perm = _run(de, mi.topk_ids, mi.topk_w, x=dev(mi.x), shared=ds)
    _check_perm(mi.topk_ids, e, True, off, perm)
    x64 = synth.bf16_to_float64(mi.x)
    _check(y, x64, mi.topk_ids, mi.topk_w, mi.experts, mi.shared, what="several permutation workgroups")
    # ids out of range: the valid pairs keep their stable order, the others go nowhere
    ids = mi.topk_ids.copy()
    bad = [(5, 3), (777, 0), (1099, 7), (1024, 2)]
    for (tt, j), v in zip(bad, (e + 1, -2, 10 ** 6, e)):
        ids[tt, j] = v
    y2, off2, perm2 = _run(de, ids, mi.topk_w, x=dev(mi.x), shared=ds)
    flat = ids.ravel().astype(np.int64)
    valid = (flat >= 0) & (flat < e)
    order = np.argsort(np.where(valid, flat, e), kind="stable")[:valid.sum()]
    exp_off = np.zeros(e + 2, np.int64)
    exp_off[1:e + 1] = np.cumsum(np.bincount(flat[valid], minlength=e))
    exp_off[e + 1] = exp_off[e] + t
    assert np.array_equal(off2, exp_off), "offsets with invalid ids"
    assert np.array_equal(perm2[:valid.sum()], order), "sorted-row order with invalid ids"
    assert np.array_equal(perm2[valid.sum():valid.sum() + t], t * k + np.arange(t)), "shared rows"
    w = mi.topk_w.copy()
    ids_ok = ids.copy()
    for tt, j in bad:
        w[tt, j] = 0
        ids_ok[tt, j] = 0
    _check(y2, x64, ids_ok, w, mi.experts, mi.shared, what="several permutation workgroups, invalid ids")


@pytest.mark.parametrize("t,h,i,e,k,routing,shared,fp4", [
    (66, 4096, 256, 100, 2, "uniform", True, False),   # shared group of 66 rows: 2 passes, each split
    (40, 4096, 512, 64, 2, "zipf", True, False),       # hot routed groups next to the shared one
    (24, 4096, 256, 48, 2, "zipf", False, True),       # fully FP4 (NVFP4 h epilogue)
])
def test_moe_decode_sized_k_split(t, h, i, e, k, routing, shared, fp4):
    """At most 2 rows per group on average and a gate/up K range of at least
    16 chunks: the K range of the groups of more than 4 rows is split 4 ways;
    the last split to finish adds the partial sums in split order, so two calls
    agree bit for bit."""
    say(f"moe decode-sized K split T={t} H={h} I={i} E={e} k={k} fp4={fp4}")
    assert h // 256 >= 16
    mi = synth.make_moe(t, h, i, e, k, seed=31, routing=routing, zipf_s=1.6, shared=shared, threads=4)
    counts = np.bincount(mi.topk_ids.ravel(), minlength=e)
    assert (t * k + (t if shared else 0)) / (e + (1 if shared else 0)) <= 2.0
    assert shared or counts.max() > 4
    de = DeviceExperts(mi.experts)
    ds = DeviceExperts(mi.shared) if shared else None
    if fp4:
        xq, xs, gs = ops.quantize_act(dev(mi.x))
        rq, rs, rgs = quant.quantize_nvfp4(mi.x.float().numpy())
        xa = quant.dequantize_nvfp4(rq, rs, rgs)
        a2 = calibrate_a2(xa, mi.topk_ids, mi.experts, range(t))
        kw = dict(x_fp4=xq, x_sf=xs, a1_gs=gs, a2_gs=f32(a2))
        x_ref = xa
    else:
        a2 = None
        kw = dict(x=dev(mi.x))
        x_ref = synth.bf16_to_float64(mi.x)
    y, off, perm = _run(de, mi.topk_ids, mi.topk_w, shared=ds, **kw)
    y2, _, _ = _run(de, mi.topk_ids, mi.topk_w, shared=ds, **kw)
    assert torch.equal(y, y2), "K-split sums differ between calls"
    _check_perm(mi.topk_ids, e, shared, off, perm)
    _check(y, x_ref, mi.topk_ids, mi.topk_w, mi.experts, mi.shared if shared else None, a2_gs=a2, x_fp4=fp4,
           what="decode-sized K split")


# ---------------------------------------------------------------------------
# full DeepSeek-V4-shaped configurations
# ---------------------------------------------------------------------------


def test_moe_decode_step_full_size():
    """MoE decode step: 64 tokens, hidden 7168, 384 experts top-8 softmax
    routing from N(0,1) logits, W1 [4096, 7168], W2 [7168, 2048], shared
    expert; every token compared."""
    say("moe decode step full size (every token)")
    de, ds = full_size_experts()
    t, e, k = 64, 384, 8
    x = synth.bf16_normal((t, 7168), 0)
    ids, w = synth.route(t, e, k, seed=0, mode="uniform")
    y, off, perm = _run(de, ids, w, x=dev(x), shared=ds)
    _check_perm(ids, e, True, off, perm)
    _check(y, synth.bf16_to_float64(x), ids, w, de.host, ds.host, what="decode, all 64 tokens")


def test_moe_prefill_chunk_full_size():
    """MoE prefill chunk: 128 tokens, Zipf(1.1)-skewed routing, shared
    expert; every token compared."""
    say("moe prefill chunk full size (every token)")
    de, ds = full_size_experts()
    t, e, k = 128, 384, 8
    x = synth.bf16_normal((t, 7168), 1)
    ids, w = synth.route(t, e, k, seed=1, mode="zipf", zipf_s=1.1)
    y, off, perm = _run(de, ids, w, x=dev(x), shared=ds)
    _check_perm(ids, e, True, off, perm)
    _check(y, synth.bf16_to_float64(x), ids, w, de.host, ds.host, what="prefill, all 128 tokens")


def test_moe_fully_fp4_large_batch_full_size():
    """Fully FP4 path: 4096 tokens quantized with gs = amax/(6*448), uniform
    top-8 routing, both GEMMs on NVFP4 activations, no shared expert.  The
    compared tokens route to every one of the 384 experts (so every group's
    work items are checked) and include the first and last token."""
    say("moe fully fp4 4096 tokens full size (tokens covering every expert)")
    de, _ = full_size_experts()
    t, e, k = 4096, 384, 8
    x = synth.bf16_normal((t, 7168), 2)
    ids, w = synth.route(t, e, k, seed=2, mode="uniform")
    xq, xs, gs = ops.quantize_act(dev(x))
    rq, rs, rgs = quant.quantize_nvfp4(x.float().numpy())
    torch.cuda.synchronize()
    assert gs.item() == float(rgs)
    assert np.array_equal(xs.cpu().numpy(), rs) and np.array_equal(xq.cpu().numpy(), rq)
    toks = covering_tokens(ids, e, extra=(0, t - 1), seed=2)
    assert len(np.unique(ids[toks])) == e
    say(f"  {len(toks)} tokens cover all {e} experts")
    xa_full = np.zeros((t, 7168))
    xa_full[toks] = quant.dequantize_nvfp4(rq[toks], rs[toks], rgs)
    # warm-up calibration of h's global scale on the first compared tokens (oracle side)
    a2 = calibrate_a2(xa_full, ids, de.host, toks[:8])
    y, off, perm = _run(de, ids, w, x_fp4=xq, x_sf=xs, a1_gs=gs, a2_gs=f32(a2))
    _check_perm(ids, e, False, off, perm)
    _check(y, xa_full, ids, w, de.host, None, tokens=toks, a2_gs=a2, x_fp4=True,
           what=f"fully fp4, {len(toks)} tokens covering all experts")
