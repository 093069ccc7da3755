"""Per-element error bound of the GPU MoE layer against the float64 oracle.

The tolerance stated for this path (normwise 2e-2 and cosine 0.999) is a
whole-tensor criterion: a wrong scale byte or a mis-indexed row whose outputs
are small can hide inside it.  This module derives, for every output element,
a bound on |y_gpu - y_ref| from the arithmetic the GPU path performs, and the
parity tests assert it beside the stated tolerance.

GPU arithmetic, in order (bf16 activations unless noted):
  1. x rows staged as fp16 after a per-row power-of-two shift that puts the
     row maximum in [2^14, 2^15): exact, except that values more than about 29
     binades below the row maximum land on fp16 subnormals (absolute error at
     most 2^-39 times the row maximum).  NVFP4 activations decode exactly.
  2. gate/up GEMM: exact products (E2M1 x E4M3 weights are exact in fp16),
     fp32 accumulation over H terms, one fp32 multiply by weight_scale_2 (times
     the activation global scale, itself one fp32 product).
  3. SwiGLU in fp32: h = g / (1 + exp(-g)) * u, exp from the hardware's
     exp2 (relative error about (2 + |g|) ulp of fp32).
  4. bf16 path: h staged as fp16 with a per-row shift (relative 2^-11, plus
     2^-39 times the row maximum for subnormals).  Fully-FP4 path: h
     quantized to NVFP4 with a2_gs, from the GPU's own fp32 h; a code or a
     block scale byte can differ from the oracle's (which quantizes its
     float64 h rounded to fp32) only where h lies within its error of a
     rounding boundary; such elements get the size of that jump.
  5. down GEMM: exact products, fp32 accumulation over I terms, one fp32
     multiply by the scales; each pair's row rounded to bf16.
  6. combine: fp32 sum of topk weighted rows then the shared row; bf16 output.

Bounds used.  Rounding to bf16 (8 significant bits) has relative error at most
u_bf16 = 2^-8 and is bounded deterministically.  Accumulation errors of the
fp32 sums follow the probabilistic model of Higham and Mary ("A new approach
to probabilistic rounding error analysis", SIAM J. Sci. Comput. 2019): the n
rounding errors delta_i are independent, zero-mean and at most u in size, so
the error sum_i delta_i s_i (s_i the partial sums) stays below
lam * u * sqrt(sum_i s_i^2) except with probability 2 exp(-lam^2 / 2)
(lam = 7: below 5e-11).  For the zero-mean synthetic operands here the
partial sums behave like a random walk over the terms t_i, whose
sum_i s_i^2 is at most about n * sum_i t_i^2, so the bound used is
lam * u * sqrt(n) * ||t||_2.  (Their worst-case form with sum|t_i| in place
of sqrt(n) * ||t||_2, about sqrt(n) = 85 times looser at K = 7168, leaves h
so uncertain that 16% of the fully-FP4 path's block scales could flip, and the
bound then checks nothing.)  The effect of the element errors of h on a
down-GEMM output is bounded the same way, by Hoeffding's inequality over the
I independent terms: lam * sqrt(sum_k (dh_k * W2[n, k])^2).  Code flips of
the fully-FP4 path (GPU and oracle on opposite sides of a rounding midpoint)
enter that sum as independent terms of random sign; a scale-byte flip moves
its 16-element block as one term.  Where the plain sum of the term bounds is
smaller than lam times their 2-norm (few terms), that deterministic sum is
used instead.  The bound is
therefore a high-probability bound under that model, not a worst case: the
worst case over every rounding in a 7168-term sum (n * u * sum|terms|) is
looser than the output values themselves and would check nothing.
"""

from __future__ import annotations

import threading

import numpy as np

from oracle import codec, moe, quant

U32 = 2.0 ** -24          # fp32 unit roundoff
U16 = 2.0 ** -11          # fp16 unit roundoff
UBF = 2.0 ** -8           # bf16 unit roundoff
SUB = 2.0 ** -38          # fp16 staging: subnormal error relative to the row maximum (2^-39, doubled)
LAM = 7.0


def _acc(n):
    """Probabilistic accumulation factor for an n-term fp32 sum (times the
    2-norm of its terms)."""
    return LAM * np.sqrt(n) * U32


class MoeBound:
    """Collects per-pair bound terms through the oracle's per-expert hook.

    o_abs[yi, j] = |o| of pair (token position yi, slot j) (slot k = shared),
    e_o[yi, j]   = bound on |GPU row before its bf16 rounding - o|."""

    def __init__(self, ntok, k, h_dim, a2_gs=None, x_fp4=False):
        self.k = k
        self.a2_gs = None if a2_gs is None else np.float32(a2_gs)
        self.x_fp4 = x_fp4
        self.o_abs = np.zeros((ntok, k + 1, h_dim))
        self.e_o = np.zeros((ntok, k + 1, h_dim))
        self.lock = threading.Lock()
        self.flips = 0

    # -- per expert ---------------------------------------------------------

    def hook(self, e, rows, a, w1d, w2d, o):
        i_dim = w1d.shape[0] // 2
        h_dim = a.shape[1]
        gu = a @ w1d.T
        g, u = gu[:, :i_dim], gu[:, i_dim:]
        aa = np.abs(a)
        # 1-2: accumulation, scale products, fp16 staging of x.  One pass over
        # W1^2 (float32 is ample for a bound) gives sum_m (a_m W1[k, m])^2 for
        # every row and, in its last row, sum_m W1[k, m]^2.
        sw1 = np.square(w1d, dtype=np.float32)
        ext = np.vstack([aa * aa, np.ones((1, h_dim))]).astype(np.float32)
        sums = (ext @ sw1.T).astype(np.float64)
        del sw1
        egu = _acc(h_dim) * np.sqrt(sums[:-1]) + 3 * U32 * np.abs(gu)
        if not self.x_fp4:
            # sum_m |W1[k, m]| <= sqrt(H) * ||W1[k]||_2
            egu += SUB * aa.max(axis=1, keepdims=True) * np.sqrt(h_dim * sums[-1])[None, :]
        eg, eu = egu[:, :i_dim], egu[:, i_dim:]
        # 3: SwiGLU in fp32 (|silu'| <= 1.1)
        sg = moe.silu(g)
        h = sg * u
        es = (4.0 + np.abs(g)) * 2.0 ** -23 * np.abs(sg)
        eh = 1.1 * eg * np.abs(u) + np.abs(sg) * eu + 1.1 * eg * eu + es * np.abs(u) + 3 * U32 * np.abs(h)
        aw2 = np.absolute(w2d, dtype=np.float32)
        f32 = lambda v: v.astype(np.float32)  # noqa: E731
        if self.a2_gs is None:
            # 4-5: fp16 h, then the down GEMM
            hmax = (np.abs(h) + eh).max(axis=1, keepdims=True)
            dh = U16 * (np.abs(h) + eh) + eh + SUB * hmax
            e_lin = np.minimum(LAM * np.sqrt((f32(dh * dh) @ np.square(aw2).T).astype(np.float64)),
                               (f32(dh) @ aw2.T).astype(np.float64))
            e_acc = _acc(i_dim) * np.sqrt((f32(np.square(np.abs(h) + dh)) @ np.square(aw2).T).astype(np.float64))
        else:
            hq, dh, blocks = self._fp4_hidden(h, eh)
            # a code flip moves one element up or down with the sign of the
            # GPU's rounding error of h: independent, zero-mean terms
            # (Hoeffding, like the fp16 rounding above); a scale-byte flip
            # moves its whole 16-element block together, so a block's effect
            # is summed first and the blocks then enter Hoeffding's sum
            e2 = (f32(dh * dh) @ np.square(aw2).T).astype(np.float64)
            e1 = (f32(dh) @ aw2.T).astype(np.float64)
            for (row, b, d16) in blocks:
                tb = (aw2[:, 16 * b:16 * b + 16] @ d16.astype(np.float32)).astype(np.float64)
                e2[row] += tb * tb
                e1[row] += tb
            # with few terms the plain sum is the tighter of the two bounds
            e_lin = np.minimum(LAM * np.sqrt(e2), e1)
            e_acc = _acc(i_dim) * np.sqrt(
                (f32(np.square(np.abs(hq) + dh + self._blk_dense(blocks, hq.shape))) @ np.square(aw2).T).astype(np.float64))
        # float32 sums of non-negative terms: relative error below 1e-3 at
        # these lengths, covered by the 1.01 factor
        e_lin = 1.01 * e_lin
        e_acc = 1.01 * e_acc.astype(np.float64)
        e_o = e_lin + e_acc + 3 * U32 * np.abs(o)
        with self.lock:
            for n, (yi, j) in enumerate(rows):
                jj = self.k if j < 0 else j
                self.o_abs[yi, jj] = np.abs(o[n])
                self.e_o[yi, jj] = e_o[n]

    def _fp4_hidden(self, h, eh):
        """Oracle's dequantized NVFP4 h, and per element the largest possible
        difference to the GPU's (zero unless a code or scale byte can flip)."""
        gs = self.a2_gs
        m, i_dim = h.shape
        h32 = h.astype(np.float32)
        hp, hs, _ = quant.quantize_nvfp4(h32, gs=gs)
        hq = quant.dequantize_nvfp4(hp, hs, gs)
        # GPU fp32 h differs from the oracle's fp32 h by at most et
        et = eh + U32 * np.abs(h) + 1e-45
        blk = lambda v: v.reshape(m, i_dim // 16, 16)  # noqa: E731
        ab = np.abs(blk(h32)).max(axis=2).astype(np.float64)
        eab = blk(et).max(axis=2)
        six_gs = float(np.float32(np.float32(6.0) * gs))
        slack = 1 + 8 * U32
        b_lo = codec.e4m3fn_encode_nonneg(np.maximum(ab - eab, 0) / six_gs / slack)
        b_hi = codec.e4m3fn_encode_nonneg((ab + eab) / six_gs * slack)
        s_lo = codec.E4M3_VALUES[b_lo] * float(gs)
        s_hi = codec.E4M3_VALUES[b_hi] * float(gs)
        byte_stable = b_lo == b_hi
        # code flips under a stable scale byte
        scale = codec.E4M3_VALUES[hs] * float(gs)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.where(scale > 0, 1.0 / scale, 0.0)
        rr = np.repeat(r, 16, axis=1)
        v = h32.astype(np.float64) * rr
        ev = et * rr * slack + np.abs(v) * 4 * U32
        c_lo = codec.e2m1_encode(v - ev)
        c_hi = codec.e2m1_encode(v + ev)
        val = codec.E2M1_VALUES
        jump = np.abs(val[c_hi] - val[c_lo]) * np.repeat(scale, 16, axis=1)
        jump = np.where(c_lo == c_hi, 0.0, np.maximum(jump, 0.0))
        # scale byte flips: every element of the block may be quantized under
        # either scale (up to twice the coarser step, plus the h error)
        unstable = np.repeat(~byte_stable, 16, axis=1)
        big = 2.0 * np.repeat(np.maximum(s_lo, s_hi), 16, axis=1) + et
        dh = np.where(unstable, 0.0, jump)
        blocks = [(int(r_), int(b_), big[r_, 16 * b_:16 * b_ + 16])
                  for r_, b_ in zip(*np.nonzero(~byte_stable))]
        with self.lock:
            self.flips += int(np.count_nonzero(dh)) + 16 * len(blocks)
        return hq, dh, blocks

    @staticmethod
    def _blk_dense(blocks, shape):
        d = np.zeros(shape)
        for (row, b, d16) in blocks:
            d[row, 16 * b:16 * b + 16] = d16
        return d

    # -- whole layer --------------------------------------------------------

    def bound(self, y_ref, topk_w, has_shared):
        """Bound on |y_gpu - y_ref| for every output element."""
        k = self.k
        w = np.abs(np.asarray(topk_w, dtype=np.float64))[:, :, None]
        s_err = UBF * (self.o_abs + self.e_o) + self.e_o          # bf16 rows
        routed = (w * s_err[:, :k]).sum(axis=1)
        mag = (w * (self.o_abs[:, :k] + s_err[:, :k])).sum(axis=1)
        if has_shared:
            routed = routed + s_err[:, k]
            mag = mag + self.o_abs[:, k] + s_err[:, k]
        y_err = routed + (k + 2) * U32 * 1.01 * mag               # fp32 combine
        return UBF * (np.abs(y_ref) + y_err) + y_err + 1e-30


def reference_and_bound(x_rows, ids, w, host, shared_host, tokens=None, a2_gs=None, x_fp4=False, workers=8):
    """Oracle output for ``tokens`` (default all) and its per-element bound."""
    ids = np.asarray(ids)
    tokens = np.arange(ids.shape[0]) if tokens is None else np.asarray(tokens)
    mb = MoeBound(len(tokens), ids.shape[1], x_rows.shape[1], a2_gs=a2_gs, x_fp4=x_fp4)
    # experts run in parallel threads; each thread's products are small, so
    # the BLAS pool is held to one thread per worker (no oversubscription)
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1 if workers > 1 else None):
        y = moe.moe_forward(x_rows, ids, w, host.expert, shared_host.expert(0) if shared_host is not None else None,
                            a2_gs=a2_gs, tokens=tokens, workers=workers, hook=mb.hook)
    wt = np.asarray(w)[tokens]
    # pairs whose expert id is invalid contribute nothing on the GPU; the
    # oracle is called with such pairs zero-weighted
    return y, mb.bound(y, wt, shared_host is not None), mb


def check_elementwise(y_gpu, y_ref, bound, what=""):
    """Assert |y_gpu - y_ref| <= bound everywhere; return the largest ratio."""
    g = np.asarray(y_gpu, dtype=np.float64)
    assert g.shape == y_ref.shape == bound.shape, (g.shape, y_ref.shape, bound.shape)
    ratio = np.abs(g - y_ref) / bound
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    r = float(ratio[worst])
    print(f"  {what}: largest error / per-element bound {r:.3f} at {tuple(int(v) for v in worst)} "
          f"(error {abs(g[worst] - y_ref[worst]):.3e}, bound {bound[worst]:.3e}, |ref| {abs(y_ref[worst]):.3e}); "
          f"median bound / |ref| {float(np.median(bound / np.maximum(np.abs(y_ref), 1e-30))):.2e}", flush=True)
    assert r <= 1.0, f"{what}: element {worst} outside its error bound ({r:.3f} x bound)"
    return r


def linear_reference_and_bound(x_rows, w_packed, w_sf, ws2, x_fp4=False):
    """Oracle output of the dense linear (x_rows: the activations' exact
    values, float64) and its per-element bound: fp16 staging of bf16 rows
    (absolute error at most 2^-39 max|x_row| per element), fp32
    accumulation of exact products (K terms, plus up to 16 K-split partial
    sums added in fp32), the scale products and the bf16 output rounding."""
    from oracle import linear
    x = np.asarray(x_rows, dtype=np.float64)
    ref = linear.linear_bf16(x, w_packed, w_sf, ws2)
    awd = np.abs(codec.dequant_nvfp4(w_packed, w_sf, ws2))
    k = x.shape[1]
    norm2 = np.sqrt((x * x) @ (awd * awd).T)
    e = _acc(k + 16) * norm2 + 3 * U32 * (np.abs(x) @ awd.T) + 3 * U32 * np.abs(ref)
    if not x_fp4:
        e += SUB * np.abs(x).max(axis=1, keepdims=True) * awd.sum(axis=1)[None, :]
    e *= 1.01
    return ref, UBF * (np.abs(ref) + e) + e + 1e-30
