"""GPU parity of nvfp4_linear and nvfp4_grouped_linear on a seeded sweep of
shapes.

The shapes are drawn once from a fixed seed (the same list on every run):
token counts from 1 (the one-launch kernel, up to 4 rows) to a few hundred
(staged activations, K splits when the work items are few, several passes),
output widths that leave partial weight-row blocks, K from 256 to 3072, bf16
and NVFP4 activations.  Dense linears are checked on every element against
the stated tolerance and their own error bound; grouped linears against the
stated tolerance."""
import numpy as np
import pytest
import torch

from gpu_util import compare, dev, f32, say
from fp4_block_scaled_route_amd import ops, synth
from moe_bound import check_elementwise, linear_reference_and_bound
from oracle import grouped_linear, linear, quant

pytestmark = pytest.mark.gpu


def _linear_shapes():
    rng = np.random.default_rng(7031)
    out = []
    for _ in range(24):
        m = int(rng.choice([1, 2, 3, 4, int(rng.integers(5, 40)), int(rng.integers(40, 260))]))
        n = 16 * int(rng.integers(1, 120))
        k = 256 * int(rng.integers(1, 13))
        out.append((m, n, k, bool(rng.random() < 0.35), int(rng.integers(0, 1 << 30))))
    return out


def _grouped_shapes():
    rng = np.random.default_rng(7032)
    out = []
    for _ in range(16):
        t = int(rng.choice([1, 2, 4, int(rng.integers(5, 70)), int(rng.integers(70, 160))]))
        g = int(rng.integers(1, 9))
        n = 16 * int(rng.integers(1, 40))
        k = 256 * int(rng.integers(1, 9))
        out.append((t, g, n, k, int(rng.integers(0, 1 << 30))))
    return out


@pytest.mark.parametrize("m,n,k,fp4,seed", _linear_shapes())
def test_linear_sweep(m, n, k, fp4, seed):
    say(f"linear sweep M={m} N={n} K={k} fp4={fp4} seed={seed}")
    li = synth.make_linear(m, n, k, seed=seed)
    if fp4:
        xq, xs, gs = ops.quantize_act(dev(li.x))
        y = ops.linear(dev(li.w), dev(li.w_sf), f32(li.ws2), x_fp4=xq, x_sf=xs, gsa=gs)
        torch.cuda.synchronize()
        rq, rs, rgs = quant.quantize_nvfp4(li.x.float().numpy())
        ref = linear.linear_nvfp4(rq, rs, rgs, li.w, li.w_sf, li.ws2)
        _, bound = linear_reference_and_bound(quant.dequantize_nvfp4(rq, rs, rgs), li.w, li.w_sf, li.ws2, x_fp4=True)
    else:
        y = ops.linear(dev(li.w), dev(li.w_sf), f32(li.ws2), x=dev(li.x))
        torch.cuda.synchronize()
        ref, bound = linear_reference_and_bound(synth.bf16_to_float64(li.x), li.w, li.w_sf, li.ws2)
    compare(y, ref, what=f"linear sweep {m}x{n}x{k}")
    check_elementwise(y.float().cpu().numpy(), ref, bound, what=f"linear sweep {m}x{n}x{k}")


@pytest.mark.parametrize("t,g,n,k,seed", _grouped_shapes())
def test_grouped_linear_sweep(t, g, n, k, seed):
    say(f"grouped linear sweep T={t} G={g} N={n} K={k} seed={seed}")
    gi = synth.make_grouped_linear(t, g, n, k, seed=seed)
    y = ops.grouped_linear(w=dev(gi.w), w_sf=dev(gi.w_sf), ws2=dev(gi.ws2), x=dev(gi.x))
    torch.cuda.synchronize()
    ref = grouped_linear.grouped_linear_bf16(synth.bf16_to_float64(gi.x), gi.w, gi.w_sf, gi.ws2)
    compare(y, ref, what=f"grouped linear sweep {t}x{g}x{n}x{k}")
