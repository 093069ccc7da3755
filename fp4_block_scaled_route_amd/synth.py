"""Seeded synthetic inputs for the NVFP4 linear and MoE workloads.

This module only draws random inputs; it holds none of the method's
arithmetic.  Both the HIP path and the CPU oracle consume what it produces.

Every tensor comes from its own numpy PCG64 stream keyed by
SeedSequence([seed, tag, index]) so that one expert's weights can be
regenerated without drawing the others, and so that the same seed gives the
same bits on any machine.

Recipe (DeepSeek-V4-style shapes):
* activations: float32 N(0, 1) rounded to bf16 (torch's round-to-nearest-even
  cast);
* packed E2M1 weights: uniform random bytes, i.e. both nibbles uniform over
  the 16 codes;
* E4M3 block scales: float32 uniform in [lo, hi] (default [0.01, 1]) rounded
  by torch's float8_e4m3fn cast (a library conversion, round to nearest even);
* weight_scale_2: a fixed value for a single linear (default 0.002), uniform
  in [0.001, 0.003] per expert for MoE layers so that mixing up experts shows;
* routing: "uniform" = top-k of N(0, 1) logits; "zipf" = Gumbel-top-k of
  log p + Gumbel noise with p_r proportional to r^-s over a seeded permutation
  of expert ranks (sampling without replacement from the Zipf law).  Routing
  weights are the softmax of the selected k logits (computed in float64,
  stored float32), so each token's weights sum to 1.
"""

from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

# stream tags
_TAG_X, _TAG_W, _TAG_SF, _TAG_WS2, _TAG_ROUTE, _TAG_PERM = 1, 2, 3, 4, 5, 6
_TAG_W1, _TAG_W1SF, _TAG_W2, _TAG_W2SF = 11, 12, 13, 14
_TAG_ROUTER = 21
_TAG_GL_X, _TAG_GL_W, _TAG_GL_SF, _TAG_GL_WS2 = 31, 32, 33, 34
_SHARED = 1 << 20   # expert index used for the shared expert's streams


def _rng(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, index])))


def bf16_normal(shape, seed: int, tag: int = _TAG_X, index: int = 0) -> torch.Tensor:
    """N(0,1) float32 draws rounded to bf16 (CPU tensor)."""
    a = _rng(seed, tag, index).standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(a).to(torch.bfloat16)


def random_bytes(shape, seed: int, tag: int, index: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(_rng(seed, tag, index).bytes(n), dtype=np.uint8).reshape(shape)


def e4m3_scales(shape, seed: int, tag: int, index: int = 0, lo: float = 0.01, hi: float = 1.0) -> np.ndarray:
    """Uniform [lo, hi] float32 draws, rounded to E4M3FN by torch's cast; bytes."""
    u = _rng(seed, tag, index).random(size=shape, dtype=np.float32)
    v = torch.from_numpy(u * np.float32(hi - lo) + np.float32(lo))
    return v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ---------------------------------------------------------------------------
# dense linear
# ---------------------------------------------------------------------------


@dataclass
class LinearInputs:
    x: torch.Tensor          # [M, K] bf16 (CPU)
    w: np.ndarray            # [N, K/2] uint8
    w_sf: np.ndarray         # [N, K/16] uint8
    ws2: float


def make_linear(m: int, n: int, k: int, seed: int = 0, ws2: float = 0.002,
                sf_range=(0.01, 1.0)) -> LinearInputs:
    if k % 16:
        raise ValueError("K must be a multiple of 16")
    x = bf16_normal((m, k), seed, _TAG_X)
    w = random_bytes((n, k // 2), seed, _TAG_W)
    sf = e4m3_scales((n, k // 16), seed, _TAG_SF, 0, *sf_range)
    return LinearInputs(x=x, w=w, w_sf=sf, ws2=float(np.float32(ws2)))


# ---------------------------------------------------------------------------
# grouped linear (attention output projection wo_a)
# ---------------------------------------------------------------------------


@dataclass
class GroupedLinearInputs:
    x: torch.Tensor          # [T, G, K] bf16 (CPU)
    w: np.ndarray            # [G, N, K/2] uint8
    w_sf: np.ndarray         # [G, N, K/16] uint8
    ws2: np.ndarray          # [G] float32


def make_grouped_linear(t: int, g: int, n: int, k: int, seed: int = 0, sf_range=(0.01, 1.0)) -> GroupedLinearInputs:
    """x ~ N(0,1) bf16; uniform codes; block scales U[0.01, 1] -> E4M3;
    per-group weight_scale_2 ~ U[0.001, 0.003] (so that a group mix-up shows)."""
    if k % 16:
        raise ValueError("K must be a multiple of 16")
    x = bf16_normal((t, g, k), seed, _TAG_GL_X)
    w = np.stack([random_bytes((n, k // 2), seed, _TAG_GL_W, i) for i in range(g)])
    sf = np.stack([e4m3_scales((n, k // 16), seed, _TAG_GL_SF, i, *sf_range) for i in range(g)])
    ws2 = (_rng(seed, _TAG_GL_WS2).random(size=g, dtype=np.float32) * np.float32(0.002)
           + np.float32(0.001)).astype(np.float32)
    return GroupedLinearInputs(x=x, w=w, w_sf=sf, ws2=ws2)


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------


def route(t: int, e: int, k: int, seed: int, mode: str = "uniform", zipf_s: float = 1.1):
    """Top-k routing from synthetic logits.  Returns (ids [T,k] int32, w [T,k] float32)."""
    rng = _rng(seed, _TAG_ROUTE)
    if mode == "uniform":
        logits = rng.standard_normal(size=(t, e))
    elif mode == "zipf":
        ranks = _rng(seed, _TAG_PERM).permutation(e) + 1          # expert -> Zipf rank
        logp = -zipf_s * np.log(ranks.astype(np.float64))
        logits = logp[None, :] + rng.gumbel(size=(t, e))
    else:
        raise ValueError(mode)
    # top-k by descending logit (continuous draws: no ties)
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, ids, axis=1)
    sel = sel - sel.max(axis=1, keepdims=True)
    w = np.exp(sel)
    w = w / w.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w.astype(np.float32)


# ---------------------------------------------------------------------------
# MoE layer
# ---------------------------------------------------------------------------


@dataclass
class ExpertSet:
    """Host copies of a stack of NVFP4 experts (routed or shared)."""
    w1: np.ndarray           # [E, 2I, H/2]
    w1_sf: np.ndarray        # [E, 2I, H/16]
    w1_ws2: np.ndarray       # [E] float32
    w2: np.ndarray           # [E, H, I/2]
    w2_sf: np.ndarray        # [E, H, I/16]
    w2_ws2: np.ndarray       # [E] float32

    def expert(self, e: int):
        return (self.w1[e], self.w1_sf[e], float(self.w1_ws2[e]),
                self.w2[e], self.w2_sf[e], float(self.w2_ws2[e]))


@dataclass
class MoEInputs:
    x: torch.Tensor                    # [T, H] bf16 (CPU)
    topk_ids: np.ndarray               # [T, k] int32
    topk_w: np.ndarray                 # [T, k] float32
    experts: ExpertSet                 # E routed experts
    shared: Optional[ExpertSet]        # 1 shared expert or None
    dims: dict = field(default_factory=dict)


def _expert_into(dst: ExpertSet, slot: int, seed: int, index: int, h: int, i: int, sf_range):
    dst.w1[slot] = random_bytes((2 * i, h // 2), seed, _TAG_W1, index)
    dst.w1_sf[slot] = e4m3_scales((2 * i, h // 16), seed, _TAG_W1SF, index, *sf_range)
    dst.w2[slot] = random_bytes((h, i // 2), seed, _TAG_W2, index)
    dst.w2_sf[slot] = e4m3_scales((h, i // 16), seed, _TAG_W2SF, index, *sf_range)


def _empty_set(n: int, h: int, i: int) -> ExpertSet:
    return ExpertSet(
        w1=np.empty((n, 2 * i, h // 2), np.uint8), w1_sf=np.empty((n, 2 * i, h // 16), np.uint8),
        w1_ws2=np.empty((n,), np.float32),
        w2=np.empty((n, h, i // 2), np.uint8), w2_sf=np.empty((n, h, i // 16), np.uint8),
        w2_ws2=np.empty((n,), np.float32))


def make_experts(n: int, h: int, i: int, seed: int, first_index: int = 0,
                 sf_range=(0.01, 1.0), threads: Optional[int] = None) -> ExpertSet:
    """n experts with stream indices first_index .. first_index+n-1."""
    s = _empty_set(n, h, i)
    ws2 = _rng(seed, _TAG_WS2, first_index).random(size=(2, n), dtype=np.float32)
    s.w1_ws2[:] = np.float32(0.001) + ws2[0] * np.float32(0.002)
    s.w2_ws2[:] = np.float32(0.001) + ws2[1] * np.float32(0.002)
    threads = threads or min(16, os.cpu_count() or 1)
    with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda e: _expert_into(s, e, seed, first_index + e, h, i, sf_range), range(n)))
    return s


def make_moe(t: int, h: int, i: int, e: int, k: int, seed: int = 0, routing: str = "uniform",
             zipf_s: float = 1.1, shared: bool = True, threads: Optional[int] = None) -> MoEInputs:
    if h % 256 or i % 256:
        raise ValueError("hidden and intermediate sizes must be multiples of 256")
    x = bf16_normal((t, h), seed, _TAG_X)
    ids, w = route(t, e, k, seed, routing, zipf_s)
    experts = make_experts(e, h, i, seed, 0, threads=threads)
    sh = make_experts(1, h, i, seed, _SHARED, threads=threads) if shared else None
    return MoEInputs(x=x, topk_ids=ids, topk_w=w, experts=experts, shared=sh,
                     dims=dict(T=t, H=h, I=i, E=e, topk=k, routing=routing))


def router_weight(e: int, h: int, seed: int, std: float = 0.05) -> torch.Tensor:
    """Router gate weight [E, H] in bf16: N(0, std^2) (a stand-in for a
    checkpoint's router weight, which is not available)."""
    w = _rng(seed, _TAG_ROUTER).standard_normal((e, h), dtype=np.float32) * np.float32(std)
    return torch.from_numpy(w).to(torch.bfloat16)


def bf16_to_float64(x: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a bf16 tensor (widening is exact)."""
    return x.to(torch.float64).numpy()
