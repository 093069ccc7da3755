"""Router gate of the MoE layer: FP8-E4M3 weight round trip, logits, top-k softmax.

Test infrastructure (the oracle): only the tests, the smoke check and the
benchmark's CPU baseline use it.

Page P1 ("commit 1121cd7"), the note on the router gate: the router weight,
once dequantized to bf16, goes through an FP8-E4M3 quantize -> dequantize round
trip with a single per-tensor scale amax/448, back to bf16, and the router is a
plain linear of the activations with that weight.  The selection feeding the
MoE layer is top-k softmax routing (k = 8 at the DeepSeek-V4 shapes).

Readings where the page is silent:
* round trip, each step one IEEE fp32 operation:
      scale = amax / 448;  byte = RNE_E4M3(w / scale) with the sign of w;
      w_r   = bf16_RNE(E4M3(byte) * scale);
* logits[t, e] = sum_k x[t, k] * w_r[e, k]: products of two bf16 values are
  exact; here they are summed in float64;
* top-k by descending logit, ties to the lower expert id;
* the k weights are the softmax of the k selected logits (so they sum to 1;
  softmax is monotone, so this equals the full softmax renormalised over the
  selected experts).
"""

import numpy as np

from . import codec

FP8_MAX = 448.0


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest even, returned as float64.

    bfloat16 keeps the top 16 bits of the float32 encoding; rounding to the
    nearest even kept pattern adds 0x7FFF plus the lowest kept bit before
    truncating (finite inputs)."""
    f = np.asarray(v, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))
    kept = ((bits + bias) >> np.uint64(16)) << np.uint64(16)
    return kept.astype(np.uint32).view(np.float32).astype(np.float64)


def fp8_scale(w: np.ndarray) -> np.float32:
    """Per-tensor FP8 scale amax / 448 (fp32)."""
    amax = np.float32(np.max(np.abs(np.asarray(w, dtype=np.float32)))) if np.size(w) else np.float32(0)
    return np.float32(amax / np.float32(FP8_MAX))


def fp8_quantize(w: np.ndarray, scale: np.float32) -> np.ndarray:
    """E4M3FN bytes of w / scale (fp32 division), nearest even, saturating at
    448, with the sign bit of w.  scale == 0 gives zeros."""
    w = np.asarray(w, dtype=np.float32)
    if scale == 0:
        return np.zeros(w.shape, dtype=np.uint8)
    q = (w / np.float32(scale)).astype(np.float32)
    mag = codec.e4m3fn_encode_nonneg(np.abs(q.astype(np.float64)))
    sign = (np.signbit(q).astype(np.uint8) << 7)
    return (mag | sign).astype(np.uint8)


def fp8_dequant_bf16(b: np.ndarray, scale: np.float32) -> np.ndarray:
    """bf16_RNE(E4M3(b) * scale), the fp32 product rounded once to bf16."""
    vals = codec.E4M3_VALUES[np.asarray(b, dtype=np.uint8)].astype(np.float32)
    return bf16_round((vals * np.float32(scale)).astype(np.float32))


def router_weight_roundtrip(w: np.ndarray):
    """The page's FP8 round trip of a bf16 router weight [E, H].
    Returns (E4M3 bytes [E, H], scale fp32, w_r [E, H] float64 holding bf16 values)."""
    scale = fp8_scale(w)
    b = fp8_quantize(w, scale)
    return b, scale, fp8_dequant_bf16(b, scale)


def topk_softmax(logits: np.ndarray, k: int):
    """Top-k of each row (descending, ties to the lower index) and the softmax
    of the selected values.  Returns (ids int32 [T, k], weights float64 [T, k])."""
    logits = np.asarray(logits, dtype=np.float64)
    t, e = logits.shape
    # sort key: descending value, then ascending index
    order = np.lexsort((np.broadcast_to(np.arange(e), (t, e)), -logits), axis=1)
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(logits, ids, axis=1)
    z = np.exp(sel - sel[:, :1])
    return ids, z / z.sum(axis=1, keepdims=True)


def route(x: np.ndarray, w_r: np.ndarray, k: int):
    """Router of tokens x [T, H] (bf16 values) with the round-tripped weight
    w_r [E, H].  Returns (logits float64 [T, E], ids int32 [T, k], weights float64 [T, k])."""
    logits = np.asarray(x, dtype=np.float64) @ np.asarray(w_r, dtype=np.float64).T
    ids, wts = topk_softmax(logits, k)
    return logits, ids, wts
