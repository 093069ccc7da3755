"""GPU parity of nvfp4_moe_grouped on a seeded sweep of small shapes.

The configurations are drawn once from a fixed seed (the list below is the
same on every run) and cover the dispatch corners of the MoE call: bf16 and
fully-FP4 activations; decode-sized batches (K-split big groups, barrier-free
small groups) and large batches (more than 16 rows per group on average: the
eight-wave kernel when K is a multiple of 1024, the four-wave one otherwise);
uniform and Zipf routing; with and without the shared expert; one expert,
top-k equal to the expert count, top-10.  Every output element is compared
with the oracle under the stated tolerance and under its own error bound, and
the permutation bit for bit."""
import numpy as np
import pytest

from gpu_util import DeviceExperts, calibrate_a2, dev, f32, say
from fp4_block_scaled_route_amd import ops, synth
from oracle import quant
from test_gpu_moe import _check, _check_perm, _run

pytestmark = pytest.mark.gpu


def _configs():
    rng = np.random.default_rng(20261203)
    out = []
    while len(out) < 32:
        e = int(rng.integers(1, 41))
        k = int(rng.integers(1, min(e, 10) + 1))
        h = 256 * int(rng.choice([1, 2, 3, 4, 5, 6, 8]))
        i = 256 * int(rng.choice([1, 2, 3, 4]))
        large = rng.random() < 0.4
        # a large batch: more than 16 rows per group on average
        t = int(rng.integers(17 * (e + 1) // k + 1, 17 * (e + 1) // k + 120)) if large else int(rng.integers(1, 96))
        if t * k > 6000:
            continue
        routing = "zipf" if rng.random() < 0.5 else "uniform"
        shared = bool(rng.random() < 0.5)
        fp4 = bool(rng.random() < 0.4)
        out.append((t, h, i, e, k, routing, shared, fp4, int(rng.integers(0, 1 << 30))))
    # corners kept explicit
    out += [
        (40, 256, 256, 1, 1, "uniform", False, False, 7),     # one expert, top-1
        (33, 512, 256, 5, 5, "uniform", True, False, 8),      # top-k = every expert
        (120, 1024, 512, 12, 10, "zipf", True, True, 9),      # top-10, fully FP4, large batch
        (200, 2048, 256, 10, 2, "zipf", False, False, 10),    # large batch, K = 2048 and 256
    ]
    return out


@pytest.mark.parametrize("t,h,i,e,k,routing,shared,fp4,seed", _configs())
def test_moe_sweep(t, h, i, e, k, routing, shared, fp4, seed):
    say(f"moe sweep T={t} H={h} I={i} E={e} k={k} {routing} shared={shared} fp4={fp4} seed={seed}")
    mi = synth.make_moe(t, h, i, e, k, seed=seed, routing=routing, shared=shared, threads=4)
    de = DeviceExperts(mi.experts)
    ds = DeviceExperts(mi.shared) if shared else None
    if fp4:
        xq, xs, gs = ops.quantize_act(dev(mi.x))
        rq, rs, rgs = quant.quantize_nvfp4(mi.x.float().numpy())
        xa = quant.dequantize_nvfp4(rq, rs, rgs)
        a2 = calibrate_a2(xa, mi.topk_ids, mi.experts, range(t), mi.shared if shared else None)
        y, off, perm = _run(de, mi.topk_ids, mi.topk_w, x_fp4=xq, x_sf=xs, a1_gs=gs, shared=ds, a2_gs=f32(a2))
        _check_perm(mi.topk_ids, e, shared, off, perm)
        _check(y, xa, mi.topk_ids, mi.topk_w, mi.experts, mi.shared if shared else None, a2_gs=a2, x_fp4=True,
               what="sweep fp4")
    else:
        y, off, perm = _run(de, mi.topk_ids, mi.topk_w, x=dev(mi.x), shared=ds)
        _check_perm(mi.topk_ids, e, shared, off, perm)
        _check(y, synth.bf16_to_float64(mi.x), mi.topk_ids, mi.topk_w, mi.experts, mi.shared if shared else None,
               what="sweep bf16")
