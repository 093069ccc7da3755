"""Number formats of NVFP4: E2M1 elements, E4M3FN block scales, nibble packing.

Weight dequantization follows page P1 ("commit 1121cd7"), the note on the
weight-dequant global scale, and page P2 ("commit efe63ca"), the notes on
weight_scale_2 being dropped and on input_scale: an NVFP4 weight element is
its E2M1 value times its FP8-E4M3 block scale times the per-tensor fp32
weight_scale_2, and nothing else.

Layout (page P2, the note on the N-major checkpoint layout and on scale
assembly): weights are stored [N, K/2] bytes with K contiguous, block scales
[N, K/16] bytes with no transpose.  Two E2M1 codes share a byte; element
2j is the low nibble and 2j+1 the high nibble (the pages do not say; this is
the usual little-endian packing and the GPU's hardware converter's order).
"""

import numpy as np

# ---------------------------------------------------------------------------
# Decoders, written from the format definitions (OCP MX v1.0).
# ---------------------------------------------------------------------------


def e2m1_decode_code(code: int) -> float:
    """Value of one 4-bit E2M1 code: sign bit 3, exponent bits 2..1 with bias 1,
    mantissa bit 0; exponent field 0 is subnormal (0 or 0.5)."""
    sign = -1.0 if code & 0b1000 else 1.0
    exp_field = (code >> 1) & 0b11
    man = code & 0b1
    if exp_field == 0:
        mag = 0.5 * man
    else:
        mag = 2.0 ** (exp_field - 1) * (1.0 + 0.5 * man)
    return sign * mag


def e4m3fn_decode_byte(b: int) -> float:
    """Value of one E4M3FN byte: sign bit 7, exponent bits 6..3 with bias 7,
    mantissa bits 2..0; exponent 0 is subnormal; S.1111.111 is NaN; no inf."""
    sign = -1.0 if b & 0x80 else 1.0
    exp_field = (b >> 3) & 0xF
    man = b & 0x7
    if exp_field == 0xF and man == 0x7:
        return float("nan")
    if exp_field == 0:
        mag = 2.0 ** -6 * (man / 8.0)
    else:
        mag = 2.0 ** (exp_field - 7) * (1.0 + man / 8.0)
    return sign * mag


#: value of every E2M1 code, float64, indexed by code 0..15
E2M1_VALUES = np.array([e2m1_decode_code(c) for c in range(16)], dtype=np.float64)
#: value of every E4M3FN byte, float64, indexed by byte 0..255 (NaN at 0x7F, 0xFF)
E4M3_VALUES = np.array([e4m3fn_decode_byte(b) for b in range(256)], dtype=np.float64)

E2M1_MAX = 6.0
E4M3_MAX = 448.0

# ---------------------------------------------------------------------------
# Encoders: round to nearest representable value, ties to the even code,
# saturating at the largest finite magnitude.  Written as "find the two
# neighbours in the sorted value table and pick the nearer", so that the rule
# is visible by eye.
# ---------------------------------------------------------------------------

# non-negative finite values and their codes, sorted ascending
_E2M1_POS_CODES = np.arange(8)
_E2M1_POS_VALUES = E2M1_VALUES[:8]            # 0, .5, 1, 1.5, 2, 3, 4, 6 (ascending)
_E4M3_POS_CODES = np.arange(0x7F)             # 0x00..0x7E: all non-negative finite
_E4M3_POS_VALUES = E4M3_VALUES[:0x7F]          # ascending


def _nearest_even(a: np.ndarray, values: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Code of the nearest entry of ``values`` (ascending, >= 0) to ``a`` (>= 0).
    Ties go to the even code.  Values beyond the last entry saturate to it."""
    a = np.asarray(a, dtype=np.float64)
    hi = np.searchsorted(values, a, side="left")          # values[hi-1] < a <= values[hi]
    hi = np.clip(hi, 0, len(values) - 1)
    lo = np.clip(hi - 1, 0, len(values) - 1)
    d_lo = np.abs(a - values[lo])
    d_hi = np.abs(values[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    out = np.where(pick_hi, codes[hi], codes[lo])
    out = np.where(a >= values[-1], codes[-1], out)       # saturate
    return out.astype(np.uint8)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even E2M1 codes of ``v`` (saturating at +-6).  The sign
    bit is the sign bit of ``v``, so -0.0 and small negatives encode as 0x8."""
    v = np.asarray(v)
    mag = _nearest_even(np.abs(v.astype(np.float64)), _E2M1_POS_VALUES, _E2M1_POS_CODES)
    sign = np.signbit(v).astype(np.uint8) << 3
    return (mag | sign).astype(np.uint8)


def e4m3fn_encode_nonneg(v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even E4M3FN byte of non-negative ``v``, saturating at
    448 (byte 0x7E).  Used for block scales, which are never negative."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(np.isnan(v)):
        raise ValueError("block scales must be non-negative numbers")
    return _nearest_even(v, _E4M3_POS_VALUES, _E4M3_POS_CODES)


# ---------------------------------------------------------------------------
# Packing and dequantization.
# ---------------------------------------------------------------------------


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes; element 2j = low nibble of byte j."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """Inverse of :func:`unpack_fp4`."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 2:
        raise ValueError("K must be even")
    return (codes[..., 0::2] & 0x0F) | ((codes[..., 1::2] & 0x0F) << 4)


def block_scales(sf: np.ndarray, k: int) -> np.ndarray:
    """[..., K/16] E4M3 bytes -> [..., K] float64 scale of every element
    (one scale per 16 consecutive elements of a row)."""
    s = E4M3_VALUES[np.asarray(sf, dtype=np.uint8)]
    if s.shape[-1] * 16 != k:
        raise ValueError("scale count does not match K/16")
    return np.repeat(s, 16, axis=-1)


def dequant_nvfp4(packed: np.ndarray, sf: np.ndarray, global_scale: float) -> np.ndarray:
    """Dequantize an NVFP4 tensor [..., K/2] + [..., K/16] to float64:
    value = E2M1(code) * E4M3(block scale) * global_scale.

    For weights the global scale is weight_scale_2 (page P1, the note on the
    weight-dequant global scale; page P2, the notes on weight_scale_2 and on
    input_scale).  For activations it is the activation global scale
    (page P3, the note on the activation global scale)."""
    codes = unpack_fp4(packed)
    k = codes.shape[-1]
    return E2M1_VALUES[codes] * block_scales(sf, k) * np.float64(global_scale)
