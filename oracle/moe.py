"""Mixture-of-Experts with NVFP4 experts: permute, expert FFN, weighted combine.

The pages describe the routed experts (Nvfp4MoE, weights stacked (E, N, K),
one weight_scale_2 per expert for each of the two layers) and a shared expert
(Nvfp4SharedExpert, its own two weight_scale_2 values) on page P2
("commit efe63ca"), the notes on weight_scale_2 being dropped and on stacking
experts on the host; the grouped GEMM taking int32 expert segment offsets on
page P3 ("commit 4c6464e"), the note on the custom-op GEMM implementation; the
gate/up projection followed by SwiGLU ("w13", the fused SwiGLU kernel) on P1
and P3; and the MoE output width being the hidden size on P3 (the note on K
being the logical width).

Readings where the pages are silent:
* routing weights are applied after the down projection and the k weighted
  expert outputs of a token are summed in order j = 0..k-1;
* the shared expert is added with weight 1;
* gate = rows [0, I) and up = rows [I, 2I) of W1; h = silu(gate) * up with
  silu(z) = z / (1 + exp(-z)); no clamp;
* segment offsets are the exclusive prefix sum of per-expert pair counts,
  length E+2: E routed groups then the shared expert's group of T rows;
  within a group rows are ordered by pair id f = t*k + j (stable).
"""

import numpy as np

from . import codec, quant


# ---------------------------------------------------------------------------
# permute / segment offsets
# ---------------------------------------------------------------------------


def permute(topk_ids: np.ndarray, num_experts: int, has_shared: bool):
    """Stable token->expert permutation.

    Returns (offsets [E+2] int32, perm [P + S*T] int32, inv [P + S*T] int32):
      offsets[e]   = number of pairs routed to experts < e
      offsets[E]   = P, offsets[E+1] = P + S*T
      perm[i]      = pair id of sorted row i (shared rows: P + t)
      inv[perm[i]] = i
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    t, k = ids.shape
    p = t * k
    flat = ids.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= num_experts):
        raise ValueError("expert id out of range")
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=num_experts)
    offsets = np.zeros(num_experts + 2, dtype=np.int64)
    offsets[1:num_experts + 1] = np.cumsum(counts)
    s = t if has_shared else 0
    offsets[num_experts + 1] = p + s
    perm = np.concatenate([order, p + np.arange(s)]) if s else order
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    return offsets.astype(np.int32), perm.astype(np.int32), inv.astype(np.int32)


# ---------------------------------------------------------------------------
# expert FFN
# ---------------------------------------------------------------------------


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def expert_ffn(a: np.ndarray, w1d: np.ndarray, w2d: np.ndarray, a2_gs=None) -> np.ndarray:
    """One expert on rows ``a`` [m, H] (float64): gate/up -> SwiGLU -> down.

    w1d: dequantized W1 [2I, H] (gate rows first), w2d: dequantized W2 [H, I].
    ``a2_gs`` not None: h is quantized to NVFP4 with that global scale (the
    float32 quantizer of ``oracle.quant``) and dequantized before the down
    projection, i.e. the down GEMM also has NVFP4 activations."""
    i = w1d.shape[0] // 2
    g = a @ w1d[:i].T
    u = a @ w1d[i:].T
    h = silu(g) * u
    if a2_gs is not None:
        hp, hs, gs = quant.quantize_nvfp4(h.astype(np.float32), gs=a2_gs)
        h = quant.dequantize_nvfp4(hp, hs, gs)
    return h @ w2d.T


def hidden_amax(a: np.ndarray, w1d: np.ndarray) -> float:
    """max |h| of the SwiGLU output for rows ``a`` (used to calibrate the
    global scale of h from a warm-up sample, page P3's calibration notes)."""
    i = w1d.shape[0] // 2
    h = silu(a @ w1d[:i].T) * (a @ w1d[i:].T)
    return float(np.max(np.abs(h.astype(np.float32)))) if h.size else 0.0


# ---------------------------------------------------------------------------
# whole MoE layer
# ---------------------------------------------------------------------------


def moe_forward(x_rows, topk_ids, topk_w, expert_weights, shared_weights=None,
                a2_gs=None, tokens=None, workers=1, hook=None):
    """y[t] = sum_j w[t, j] * FFN_{ids[t, j]}(x_t) + FFN_shared(x_t), float64.

    x_rows:   [T, H] float64 activations as the experts see them (bf16 values,
              or dequantized NVFP4 activations for the fully-FP4 path).
    expert_weights(e) -> (w1 packed [2I, H/2], w1 sf [2I, H/16], ws2_1,
                          w2 packed [H, I/2],  w2 sf [H, I/16],  ws2_2)
    shared_weights: same tuple for the shared expert, or None.
    tokens:   subset of token indices to compute (default: all).  Experts are
              dequantized one at a time to bound host memory.
    workers:  experts evaluated concurrently by that many threads (each expert's
              result is independent; the combine below runs afterwards in
              the fixed order, so the result does not depend on it).
    hook:     optional callable hook(e, rows, a, w1d, w2d, o) run once per
              evaluated expert (e = -1 for the shared expert) with the output
              positions ``rows`` (index into ``tokens``) and j of its pairs
              (j = -1 for the shared expert), its input rows ``a``, its
              dequantized weights and its output rows ``o``; test code uses it
              to derive error bounds
              from the same weights.  It must not modify its arguments.
    Returns y [len(tokens), H] float64 in the order of ``tokens``."""
    ids = np.asarray(topk_ids)
    w = np.asarray(topk_w, dtype=np.float64)
    t_all = ids.shape[0]
    tokens = np.arange(t_all) if tokens is None else np.asarray(tokens)
    h_dim = x_rows.shape[1]
    y = np.zeros((len(tokens), h_dim), dtype=np.float64)
    pos = {int(t): n for n, t in enumerate(tokens)}
    # per expert: which (row of y, j) pairs use it
    uses = {}
    for t in tokens:
        for j in range(ids.shape[1]):
            uses.setdefault(int(ids[t, j]), []).append((pos[int(t)], int(t), j))
    # accumulate per pair into a [len(tokens), k] table first so that the sum
    # over j runs in order j = 0..k-1 for every token
    k = ids.shape[1]
    outs = np.zeros((len(tokens), k, h_dim), dtype=np.float64)

    def one_expert(e):
        w1, s1, g1, w2, s2, g2 = expert_weights(e)
        w1d = codec.dequant_nvfp4(w1, s1, g1)
        w2d = codec.dequant_nvfp4(w2, s2, g2)
        rows = uses[e]
        a = np.stack([x_rows[t] for (_, t, _) in rows]).astype(np.float64)
        o = expert_ffn(a, w1d, w2d, a2_gs)
        for n, (yi, _, j) in enumerate(rows):
            outs[yi, j] = o[n]
        if hook is not None:
            hook(e, [(yi, j) for (yi, _, j) in rows], a, w1d, w2d, o)

    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one_expert, sorted(uses)))
    else:
        for e in sorted(uses):
            one_expert(e)
    for j in range(k):
        y += w[tokens, j][:, None] * outs[:, j]
    if shared_weights is not None:
        w1, s1, g1, w2, s2, g2 = shared_weights
        w1d = codec.dequant_nvfp4(w1, s1, g1)
        w2d = codec.dequant_nvfp4(w2, s2, g2)
        a = np.asarray(x_rows[tokens], dtype=np.float64)
        o = expert_ffn(a, w1d, w2d, a2_gs)
        y += o
        if hook is not None:
            hook(-1, [(yi, -1) for yi in range(len(tokens))], a, w1d, w2d, o)
    return y
