"""Helpers shared by the GPU parity tests: device upload of synthetic inputs,
the comparison rule, and a once-per-session full-size expert set."""
import os
import sys

import numpy as np
import torch

from fp4_block_scaled_route_amd import synth

# bf16 outputs vs the float64 oracle: normwise max |gpu - ref| / max |ref| and
# cosine similarity (the tolerance stated for this path: 2e-2 and 0.999).
TOL_REL = 2e-2
TOL_COS = 0.999


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    t = a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda()


def f32(v):
    return torch.tensor([float(v)], dtype=torch.float32, device="cuda")


def compare(y_gpu, ref, tol=TOL_REL, cos_min=TOL_COS, what=""):
    g = y_gpu.float().cpu().numpy().astype(np.float64) if isinstance(y_gpu, torch.Tensor) else y_gpu
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    scale = np.abs(ref).max()
    err = np.abs(g - ref).max() / scale if scale > 0 else np.abs(g).max()
    cos = float((g * ref).sum() / (np.linalg.norm(g) * np.linalg.norm(ref))) if scale > 0 else 1.0
    say(f"  {what}: normwise max rel err {err:.3e}, cos {cos:.6f}")
    assert err <= tol, f"{what}: normwise error {err} > {tol}"
    assert cos >= cos_min, f"{what}: cosine {cos} < {cos_min}"
    return err, cos


class DeviceExperts:
    """Device copies of an ExpertSet (stacked) plus the host copy for the oracle."""

    def __init__(self, host: "synth.ExpertSet"):
        self.host = host
        self.w1 = dev(host.w1)
        self.w1_sf = dev(host.w1_sf)
        self.w1_ws2 = dev(host.w1_ws2)
        self.w2 = dev(host.w2)
        self.w2_sf = dev(host.w2_sf)
        self.w2_ws2 = dev(host.w2_ws2)

    def args(self):
        return dict(w1=self.w1, w1_sf=self.w1_sf, w1_ws2=self.w1_ws2,
                    w2=self.w2, w2_sf=self.w2_sf, w2_ws2=self.w2_ws2)

    def as_shared(self):
        return (self.w1[0], self.w1_sf[0], self.w1_ws2[:1], self.w2[0], self.w2_sf[0], self.w2_ws2[:1])


_FULL = {}


def full_size_experts(seed=0, h=7168, i=2048, e=384):
    """The DeepSeek-V4-shaped expert stack (384 experts, W1 [4096, 7168],
    W2 [7168, 2048]) and one shared expert, generated and uploaded once."""
    key = (seed, h, i, e)
    if key not in _FULL:
        say(f"  generating {e} experts H={h} I={i} seed={seed}")
        routed = synth.make_experts(e, h, i, seed, 0)
        shared = synth.make_experts(1, h, i, seed, synth._SHARED)
        _FULL[key] = (DeviceExperts(routed), DeviceExperts(shared))
    return _FULL[key]


def calibrate_a2(xa, ids, host, tokens, shared_host=None, workers=16):
    """Oracle-side warm-up calibration of the hidden activations' global
    scale: max |h| over the pairs of ``tokens`` / 2688 (float32), each
    expert's W1 dequantized once."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import codec, moe
    rows = {}
    for t in tokens:
        for j in range(ids.shape[1]):
            rows.setdefault(int(ids[t, j]), []).append(int(t))

    def one(e):
        src = host.expert(e) if e >= 0 else shared_host.expert(0)
        r = rows[e] if e >= 0 else [int(t) for t in tokens]
        return moe.hidden_amax(np.asarray(xa[r], dtype=np.float64), codec.dequant_nvfp4(*src[:3]))

    keys = sorted(rows) + ([-1] if shared_host is not None else [])
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers) as ex:
        amax = max(ex.map(one, keys))
    return np.float32(np.float32(amax) / np.float32(2688.0))


def covering_tokens(ids, n_experts, extra=(), seed=0, per_expert=1):
    """Tokens whose routed experts cover every expert (greedy set cover over
    a seeded shuffle of the batch), plus ``extra``; sorted."""
    rng = np.random.default_rng(seed)
    need = {e: per_expert for e in range(n_experts)}
    chosen = set(int(v) for v in extra)
    for t in chosen:
        for e in ids[t]:
            if need.get(int(e), 0) > 0:
                need[int(e)] -= 1
    for t in rng.permutation(ids.shape[0]):
        if not any(v > 0 for v in need.values()):
            break
        gain = sum(1 for e in ids[t] if need.get(int(e), 0) > 0)
        if gain >= 2 or (gain == 1 and len(chosen) > 4 * n_experts // ids.shape[1]):
            chosen.add(int(t))
            for e in ids[t]:
                if need.get(int(e), 0) > 0:
                    need[int(e)] -= 1
    for e, v in need.items():   # any expert still missing: its first token
        if v > 0:
            chosen.add(int(np.nonzero((ids == e).any(axis=1))[0][0]))
    return sorted(chosen)
