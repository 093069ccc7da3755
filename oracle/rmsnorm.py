"""RMSNorm fused with the NVFP4 activation quantization (the "P4" fusion).

Test infrastructure (the oracle): only the tests, the smoke check and the
benchmark's CPU baseline use it.

Page P1 ("commit 1121cd7 - single_shot_inference.py"), the notes on the A/B
comparison of the fused and unfused paths: the fused RMSNorm + NVFP4
quantization ("P4") feeds the q_a and kv projections, and its activation
global scale, FP4 data and GEMM outputs must match the unfused path (RMSNorm,
then quantize_activation_nvfp4); the page records a correctness regression
of that fusion.  So the fused operation is defined as the composition: the
quantizer (oracle/quant.py) applied to the RMSNorm output.

RMSNorm itself is not spelled out on the pages.  Reading (the usual RMSNorm
with a learned weight, each rounding stated so that codes are reproducible):

  ss  = sum_k x[k]^2            float64 (each square of a bf16 value is exact)
  r   = float32(1 / sqrt(ss / K + eps))     float64 operations, one rounding
  y_k = bf16_RNE(float32(float32(x_k * r) * w_k))

The unfused path rounds its output to bf16 before the quantizer reads it, so
the fused path quantizes these bf16 values (not the float32 products).
"""

import numpy as np

from . import quant


def bf16_round(v: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16, round to nearest even (finite values), as float32."""
    f = np.asarray(v, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))
    kept = ((bits + bias) >> np.uint64(16)) << np.uint64(16)
    return kept.astype(np.uint32).view(np.float32)


def rms_scale(x: np.ndarray, eps: float) -> np.ndarray:
    """r per row: float32(1 / sqrt(mean(x^2) + eps)), the mean and root in float64."""
    x = np.asarray(x, dtype=np.float64)
    ss = np.sum(x * x, axis=-1)
    return (1.0 / np.sqrt(ss / x.shape[-1] + float(np.float32(eps)))).astype(np.float32)


def rmsnorm_bf16(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of rows x [T, K] (bf16 values) with weight w [K] (bf16 values):
    bf16 values returned as float32."""
    x32 = np.asarray(x, dtype=np.float32)
    r = rms_scale(x32, eps)
    xr = (x32 * r[:, None]).astype(np.float32)
    return bf16_round((xr * np.asarray(w, dtype=np.float32)[None, :]).astype(np.float32))


def rmsnorm_quantize(x: np.ndarray, w: np.ndarray, eps: float, gs=None):
    """The fused operation: (y, packed codes, scale bytes, gs) with y the RMSNorm
    output and the rest nvfp4 quantization of y (gs computed from y when None)."""
    y = rmsnorm_bf16(x, w, eps)
    packed, sbytes, g = quant.quantize_nvfp4(y, gs)
    return y, packed, sbytes, g
