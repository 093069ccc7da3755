"""NVFP4 activation quantization, float32, fixed operation order.

Page P3 ("commit 4c6464e"), the note on the activation global scale: the
activation global scale is gs = amax / (6 * 448), where 6 is the largest E2M1
magnitude and 448 the largest E4M3 magnitude, and gs is used as it is (it is
not inverted).  The same page's notes on warm-up calibration say gs comes from
the actual activation distribution.  Page P3's description of the MoE and
linear GEMM implementation names the quantizer (quantize_activation_nvfp4)
but not its internals; the per-block steps below are the plainest reading
that keeps every code within +-6 and every scale within 448:

  amax  = max |x|                      (whole tensor)
  gs    = amax / 2688                  (2688 = 6 * 448)
  per 16-element block of a row:
    ab    = max |x_blk|
    sf    = ab / (6 * gs)             -> byte = RNE_E4M3(sf), saturating
    scale = E4M3(byte) * gs
    if scale == 0: every code is 0
    else:          r = 1 / scale;  code = RNE_E2M1(x * r), saturating at 6

Every step is one IEEE float32 operation (round to nearest even), exactly in
this order; the GPU kernel performs the same operations, so codes and scale
bytes agree bit for bit.  When gs == 0 (an all-zero tensor) every scale byte
and code is 0.
"""

import numpy as np

from . import codec

F32 = np.float32
GS_DIVISOR = F32(6.0 * 448.0)   # 2688, exact in float32


def global_scale(x: np.ndarray) -> np.float32:
    """gs = amax / (6*448) in float32 (page P3, note on the activation global scale)."""
    x = np.asarray(x, dtype=F32)
    amax = F32(np.max(np.abs(x))) if x.size else F32(0.0)
    return F32(amax / GS_DIVISOR)


def quantize_nvfp4(x: np.ndarray, gs=None):
    """Quantize float32 activations [M, K] (K % 16 == 0) to NVFP4.

    Returns (packed codes [M, K/2] uint8, scale bytes [M, K/16] uint8, gs float32).
    ``gs`` None means "compute it from x" (the per-tensor amax rule)."""
    x = np.asarray(x, dtype=F32)
    if x.ndim != 2 or x.shape[1] % 16:
        raise ValueError("x must be [M, K] with K a multiple of 16")
    m, k = x.shape
    gs = global_scale(x) if gs is None else F32(gs)
    blocks = x.reshape(m, k // 16, 16)
    ab = np.max(np.abs(blocks), axis=2)                         # float32, exact
    if gs == 0:
        sbytes = np.zeros((m, k // 16), dtype=np.uint8)
    else:
        denom = F32(F32(6.0) * gs)
        sf = (ab / denom).astype(F32)                           # one float32 division
        sbytes = codec.e4m3fn_encode_nonneg(sf)
    s_dec = codec.E4M3_VALUES[sbytes].astype(F32)               # exact in float32
    scale = (s_dec * gs).astype(F32)                            # one float32 product
    codes = np.zeros((m, k // 16, 16), dtype=np.uint8)
    nz = scale != 0
    if np.any(nz):
        r = np.zeros_like(scale)
        r[nz] = (F32(1.0) / scale[nz]).astype(F32)              # one float32 division
        v = (blocks * r[:, :, None]).astype(F32)                # one float32 product
        enc = codec.e2m1_encode(v)
        codes = np.where(nz[:, :, None], enc, np.uint8(0)).astype(np.uint8)
    packed = codec.pack_fp4(codes.reshape(m, k))
    return packed, sbytes, gs


def dequantize_nvfp4(packed: np.ndarray, sbytes: np.ndarray, gs) -> np.ndarray:
    """float64 values E2M1(code) * E4M3(scale) * gs of a quantized tensor."""
    return codec.dequant_nvfp4(packed, sbytes, float(F32(gs)))
