"""NVFP4 grouped linear of the attention output projection (wo_a), float64.

Test infrastructure (the oracle): only the tests, the smoke check and the
benchmark's CPU baseline use it.

Page P3 ("commit 4c6464e - vllm"), the notes on the BF16 wo_a path (the
grouped shapes of the BMM) and on replacing the wo_a path with an NVFP4
grouped linear: wo_a is a batched matmul over n_local_groups = 8
groups whose input features per group are n_heads * head_dim / n_groups =
4096; the tokens' [T, 8 * 4096] activations are viewed as [T, 8, 4096] and
group g is multiplied by its own weight (einsum 'bhr,hdr->bhd':
y[t, g, d] = sum_r x[t, g, r] * W[g, d, r]); the pages replace it with an
NVFP4 grouped GEMM over the 8 groups.

Readings where the pages are silent:
* the output width per group (d) is not on the pages; the workloads use 1024,
  the tests several widths;
* every group's weight is NVFP4 ([N, K/2] codes, [N, K/16] E4M3 block scales)
  with its own weight_scale_2 (a [G] vector), applied as in the dense linear;
* the activations are bf16 (the pages feed wo_a the bf16 output of the
  inverse RoPE), or NVFP4 with one activation global scale for the whole
  [T, G, K] tensor (the dense linear's convention);
* output layout [T, G, d] (the einsum's), bf16.
"""

import numpy as np

from . import codec


def grouped_linear_bf16(x: np.ndarray, w_packed: np.ndarray, w_sf: np.ndarray, ws2: np.ndarray) -> np.ndarray:
    """x [T, G, K] (exact bf16 values), w_packed [G, N, K/2], w_sf [G, N, K/16],
    ws2 [G].  Returns y [T, G, N] = einsum('tgk,gnk->tgn', x, Wd), float64."""
    x = np.asarray(x, dtype=np.float64)
    g_count = w_packed.shape[0]
    wd = np.stack([codec.dequant_nvfp4(w_packed[g], w_sf[g], float(ws2[g])) for g in range(g_count)])
    return np.einsum("tgk,gnk->tgn", x, wd)


def grouped_linear_nvfp4(x_packed, x_sf, gsa, w_packed, w_sf, ws2) -> np.ndarray:
    """NVFP4 activations x_packed [T, G, K/2], x_sf [T, G, K/16] with one global
    scale gsa: the same product on the dequantized activations."""
    t, g_count, kh = x_packed.shape
    xd = codec.dequant_nvfp4(x_packed.reshape(t * g_count, kh), x_sf.reshape(t * g_count, -1), gsa)
    return grouped_linear_bf16(xd.reshape(t, g_count, 2 * kh), w_packed, w_sf, ws2)
