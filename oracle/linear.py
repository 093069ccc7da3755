"""Dense NVFP4 block-scaled linear, float64.

Page P1 ("commit 1121cd7"), the note on the weight-dequant global scale,
states the GEMM as y = (x * scale_a * gsa) @ (w * scale_b * gsb): each operand
is its E2M1 values times its E4M3 block scales times its global scale, and y
is the plain matrix product of the two dequantized operands (W is [N, K] so
the product is x @ W^T).  The global-scale wiring is read as follows (pages
P1/P2/P3 disagree; see the notes on input_scale on P2 and on the activation
global scale on P3): the weight side carries weight_scale_2 only, the
activation side carries the activation global scale, and the product of the
two is applied exactly once.  With bf16 activations scale_a = gsa = 1.
"""

import numpy as np

from . import codec


def linear_bf16(x: np.ndarray, w_packed: np.ndarray, w_sf: np.ndarray, ws2: float) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * Wd[n, k] in float64, Wd = dequantized weights.
    ``x`` holds the activations' exact values (bf16 values widened)."""
    wd = codec.dequant_nvfp4(w_packed, w_sf, ws2)               # [N, K] float64
    return np.asarray(x, dtype=np.float64) @ wd.T


def linear_nvfp4(x_packed, x_sf, gsa, w_packed, w_sf, ws2) -> np.ndarray:
    """Both operands NVFP4: y = (E2M1(x) * E4M3(sx) * gsa) @ (E2M1(w) * E4M3(sw) * ws2)^T."""
    xd = codec.dequant_nvfp4(x_packed, x_sf, gsa)
    wd = codec.dequant_nvfp4(w_packed, w_sf, ws2)
    return xd @ wd.T
