"""GPU parity of the router gate (nvfp4_router_prepare / nvfp4_router_topk)
against the oracle (oracle/router.py).

* The weight preparation is bit-exact: the FP8 round trip is a chain of
  correctly rounded fp32 operations on both sides.
* Logits: the GPU accumulates exact bf16 products in fp32, the oracle in
  float64; they agree within the fp32 dot-product bound K * 2^-24 * sum|x w|.
* Selection: floating point decides the integer ids, so both sides decide in
  the GPU's precision: the oracle's top-k softmax applied to the GPU's own
  logits must give the same ids bit for bit, and the weights within fp32
  rounding.  Against the oracle's own float64 logits the ids agree wherever
  the k-th and (k+1)-th logits are further apart than twice the largest logit
  difference of that row.
"""
import numpy as np
import pytest
import torch

from gpu_util import dev, say
from fp4_block_scaled_route_amd import ops, synth
from oracle import router

pytestmark = pytest.mark.gpu


def _inputs(t, h, e, seed):
    x = synth.bf16_normal((t, h), seed)
    w = torch.from_numpy(np.random.default_rng(seed + 100).standard_normal((e, h)).astype(np.float32) * 0.05)
    return x, w.to(torch.bfloat16)


def _check(t, h, e, k, seed):
    x, w = _inputs(t, h, e, seed)
    wr_gpu, scale = ops.router_prepare(dev(w))
    b, scale_ref, wr_ref = router.router_weight_roundtrip(w.float().numpy())
    torch.cuda.synchronize()
    assert scale.item() == float(scale_ref)
    assert np.array_equal(wr_gpu.cpu().double().numpy(), wr_ref), "round-tripped weight differs"
    logits, ids, wts = ops.router_topk(dev(x), wr_gpu, k)
    torch.cuda.synchronize()
    lg = logits.cpu().double().numpy()
    xf = synth.bf16_to_float64(x)
    ref_lg, ref_ids, _ = router.route(xf, wr_ref, k)
    bound = h * 2.0 ** -24 * (np.abs(xf) @ np.abs(wr_ref).T) + 1e-30
    err = np.abs(lg - ref_lg)
    say(f"  router T={t} H={h} E={e} k={k}: max |dlogit|/bound {float((err / bound).max()):.3f}")
    assert np.all(err <= bound)
    # selection in the GPU's precision
    sel_ids, sel_w = router.topk_softmax(lg, k)
    assert np.array_equal(ids.cpu().numpy(), sel_ids)
    assert np.allclose(wts.cpu().double().numpy(), sel_w, rtol=2e-6, atol=1e-7)
    # against float64 logits, in the rows whose k-th/(k+1)-th margin exceeds
    # twice that row's largest logit difference (elsewhere either order is a
    # correct rounding of the same sum)
    srt = -np.sort(-ref_lg, axis=1)
    margin = srt[:, k - 1] - srt[:, k] if k < e else np.full(t, np.inf)
    clear = margin > 2 * err.max(axis=1)
    say(f"    rows with a clear k-th margin: {int(clear.sum())}/{t}")
    assert clear.mean() > 0.5
    assert np.array_equal(ids.cpu().numpy()[clear], ref_ids[clear])


@pytest.mark.parametrize("t,h,e,k", [
    (1, 256, 16, 4),
    (37, 512, 40, 3),        # ragged token and expert tiles
    (64, 7168, 384, 8),      # decode step
    (300, 1024, 512, 64),    # largest expert count and selection
])
def test_router_parity(t, h, e, k):
    say(f"router parity T={t} H={h} E={e} k={k}")
    _check(t, h, e, k, seed=t + e)


def test_router_ties_go_to_the_lower_id():
    # identical expert rows give identical logits: the lower ids must win
    t, h, e, k = 8, 256, 32, 4
    x, w = _inputs(t, h, e, 3)
    w[5:12] = w[5]
    wr, _ = ops.router_prepare(dev(w))
    logits, ids, wts = ops.router_topk(dev(x), wr, k)
    torch.cuda.synchronize()
    sel_ids, _ = router.topk_softmax(logits.cpu().double().numpy(), k)
    assert np.array_equal(ids.cpu().numpy(), sel_ids)


def test_router_feeds_the_moe_layer():
    """The router's outputs are valid routing inputs: distinct ids in [0, E),
    weights summing to 1."""
    t, h, e, k = 64, 512, 48, 8
    x, w = _inputs(t, h, e, 9)
    wr, _ = ops.router_prepare(dev(w))
    _, ids, wts = ops.router_topk(dev(x), wr, k)
    torch.cuda.synchronize()
    ids = ids.cpu().numpy()
    assert ids.min() >= 0 and ids.max() < e
    assert all(len(set(r)) == k for r in ids)
    assert np.allclose(wts.cpu().numpy().sum(1), 1.0, atol=1e-5)


def test_router_prepare_zero_weight():
    w = torch.zeros((16, 256), dtype=torch.bfloat16)
    wr, scale = ops.router_prepare(dev(w))
    torch.cuda.synchronize()
    assert scale.item() == 0.0 and not wr.any().item()
