"""GPU parity of nvfp4_grouped_linear (attention output projection wo_a)
against the float64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from gpu_util import compare, dev, say
from fp4_block_scaled_route_amd import ops, synth
from oracle import grouped_linear, quant

pytestmark = pytest.mark.gpu


def _inputs(t, g, n, k, seed=0):
    gi = synth.make_grouped_linear(t, g, n, k, seed=seed)
    return gi, dict(w=dev(gi.w), w_sf=dev(gi.w_sf), ws2=dev(gi.ws2))


@pytest.mark.parametrize("t,g,n,k", [
    (1, 8, 64, 512), (4, 8, 128, 512),          # one-launch kernel (up to 4 rows per group)
    (2, 8, 1024, 4096),                         # the same at the decode shape's K and width
    (5, 8, 128, 1024), (37, 8, 96, 1024),       # four-wave kernel; partial weight-row block
    (20, 3, 64, 768),                           # K not a multiple of 1024
    (64, 8, 1024, 4096),                        # decode shape: 8 groups, K 4096, width 1024
    (130, 3, 64, 1024), (300, 2, 48, 2048),     # eight-wave kernel, several passes, ragged tail
])
def test_grouped_linear_bf16(t, g, n, k):
    say(f"grouped linear bf16 T={t} G={g} N={n} K={k}")
    gi, w = _inputs(t, g, n, k)
    y = ops.grouped_linear(**w, x=dev(gi.x))
    torch.cuda.synchronize()
    ref = grouped_linear.grouped_linear_bf16(synth.bf16_to_float64(gi.x), gi.w, gi.w_sf, gi.ws2)
    compare(y, ref, what=f"grouped linear {t}x{g}x{n}x{k}")


@pytest.mark.parametrize("t", [3, 64, 200])
def test_grouped_linear_nvfp4_activations(t):
    g, n, k = 8, 128, 1024
    say(f"grouped linear NVFP4 activations T={t}")
    gi, w = _inputs(t, g, n, k, seed=1)
    xq, xs, gs = ops.quantize_act(dev(gi.x).reshape(t * g, k))
    y = ops.grouped_linear(**w, x_fp4=xq.reshape(t, g, k // 2), x_sf=xs.reshape(t, g, k // 16), gsa=gs)
    torch.cuda.synchronize()
    # the oracle quantizes the same activations itself (bit-exact quantizer)
    packed, sbytes, gso = quant.quantize_nvfp4(gi.x.float().numpy().reshape(t * g, k))
    assert np.array_equal(xq.cpu().numpy(), packed) and np.array_equal(xs.cpu().numpy(), sbytes)
    ref = grouped_linear.grouped_linear_nvfp4(packed.reshape(t, g, k // 2), sbytes.reshape(t, g, k // 16), gso,
                                              gi.w, gi.w_sf, gi.ws2)
    compare(y, ref, what=f"grouped linear NVFP4 T={t}")


def test_grouped_linear_full_batch_sampled_tokens():
    """4096 tokens x 8 groups x width 1024 x K 4096 (the eight-wave launch);
    the oracle computes a sample of tokens (rows are independent)."""
    t, g, n, k = 4096, 8, 1024, 4096
    say("grouped linear 4096 tokens, sampled rows")
    gi, w = _inputs(t, g, n, k, seed=2)
    y = ops.grouped_linear(**w, x=dev(gi.x))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 111, 112, 2047, 3999, 4095])
    ref = grouped_linear.grouped_linear_bf16(synth.bf16_to_float64(gi.x[rows]), gi.w, gi.w_sf, gi.ws2)
    compare(y[rows], ref, what="grouped linear 4096 sampled")


def test_grouped_linear_group_order_and_zero_tokens():
    """Each group uses its own weight and weight_scale_2: zeroing one group's
    ws2 zeroes exactly that group's outputs; T = 0 writes nothing."""
    t, g, n, k = 6, 8, 64, 512
    gi, w = _inputs(t, g, n, k, seed=3)
    ws2 = w["ws2"].clone()
    ws2[5] = 0.0
    y = ops.grouped_linear(w["w"], w["w_sf"], ws2, x=dev(gi.x)).float().cpu()
    assert not y[:, 5].any()
    assert (y[:, [0, 1, 2, 3, 4, 6, 7]].abs().sum(dim=(0, 2)) > 0).all()
    empty = torch.full((0, g, n), 7.0, dtype=torch.bfloat16, device="cuda")
    ops.grouped_linear(**w, x=torch.empty((0, g, k), dtype=torch.bfloat16, device="cuda"), out=empty)
    torch.cuda.synchronize()
