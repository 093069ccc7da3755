#!/usr/bin/env python3
"""Benchmark of the NVFP4 MoE layer (and dense linear) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of seeded synthetic
input that is already resident in HBM: for the MoE workloads one
nvfp4_moe_grouped call (permute, gate/up GEMM + SwiGLU, down GEMM + scatter,
weighted combine), preceded by nvfp4_quantize_act on the fully-FP4 workload.
Prints ONE JSON line.

Default (no --workload): the headline line is the fully-FP4 MoE batch (4096
tokens, both GEMMs on NVFP4 activations), the configuration at the bf16
MFMA ridge: `value` is its step throughput in TFLOP/s, reported with and
without the activation quantizer; the MoE decode step (64 tokens) and
prefill chunk (128 tokens, Zipf routing) are nested under "configs", each
with its own ms_per_step, roofline and CPU oracle baseline.  All three use
the same 384-expert stack.  The roofline objects describe each step's
dominant kernel (the gate/up GEMM), timed with HIP events recorded around it
on the stream it runs on.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
FP16_PEAK_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA
BF16_RIDGE_FLOP_PER_BYTE = FP16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # 312.5
BYTES_PER_EXPERT_W1 = 2 * 2048 * 7168 // 2 + 2 * 2048 * 7168 // 16       # 16,515,072
BYTES_PER_EXPERT_W2 = 7168 * 2048 // 2 + 7168 * 2048 // 16               # 8,257,536
FLOPS_PER_PAIR = 2 * (2 * 2048 * 7168 + 7168 * 2048)                     # 88,080,384

WORKLOADS = {
    # MoE decode step: 64 tokens, 384 experts, top-8 softmax routing, shared expert
    "moe_decode": dict(kind="moe", T=64, H=7168, I=2048, E=384, k=8, routing="uniform", shared=True, fp4=False),
    # MoE prefill chunk: 128 tokens, Zipf(1.1) routing, shared expert
    "moe_prefill": dict(kind="moe", T=128, H=7168, I=2048, E=384, k=8, routing="zipf", shared=True, fp4=False),
    # fully FP4 path: 4096 tokens, both GEMMs on NVFP4 activations, no shared expert
    "moe_fp4": dict(kind="moe", T=4096, H=7168, I=2048, E=384, k=8, routing="uniform", shared=False, fp4=True),
    # router gate (FP8 round-tripped bf16 weight, top-8 softmax) at the decode and large-batch token counts
    "router_decode": dict(kind="router", T=64, H=7168, E=384, k=8),
    "router_4096": dict(kind="router", T=4096, H=7168, E=384, k=8),
    # RMSNorm fused with the NVFP4 activation quantization (feeds the q_a / kv projections)
    "rmsnorm_quant_decode": dict(kind="rmsnorm_quant", T=64, K=7168),
    "rmsnorm_quant_4096": dict(kind="rmsnorm_quant", T=4096, K=7168),
    # attention output projection wo_a: 8 groups of K 4096, output width 1024 per group
    "wo_a_decode": dict(kind="grouped_linear", T=64, G=8, N=1024, K=4096),
    "wo_a_4096": dict(kind="grouped_linear", T=4096, G=8, N=1024, K=4096),
    # dense NVFP4 linear: the small single-linear check shape, then the projection shapes
    "linear_small": dict(kind="linear", M=8, N=128, K=256),
    "linear_q_a_m1": dict(kind="linear", M=1, N=1536, K=7168),
    "linear_q_a_m32": dict(kind="linear", M=32, N=1536, K=7168),
    "linear_q_a_m128": dict(kind="linear", M=128, N=1536, K=7168),
    "linear_q_b_m1": dict(kind="linear", M=1, N=24576, K=1536),
    "linear_q_b_m32": dict(kind="linear", M=32, N=24576, K=1536),
    "linear_q_b_m128": dict(kind="linear", M=128, N=24576, K=1536),
}


def cpu_model():
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (the library records them on the stream its
    kernels run on)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(ev.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp4_block_scaled_route_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload, src_hash):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"gate_up_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_hash") != src_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# MoE workload
# ---------------------------------------------------------------------------


class ExpertStack:
    """One layer's routed experts and shared expert, on the host (for the
    oracle) and on the device; shared by every MoE workload of a run."""

    def __init__(self, cfg, seed):
        import numpy as np
        import torch

        from fp4_block_scaled_route_amd import synth

        t0 = time.time()
        self.key = (cfg["E"], cfg["H"], cfg["I"], seed)
        self.routed = synth.make_experts(cfg["E"], cfg["H"], cfg["I"], seed, 0)
        self.shared = synth.make_experts(1, cfg["H"], cfg["I"], seed, synth._SHARED)
        d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
        ex, s = self.routed, self.shared
        self.dev = dict(w1=d(ex.w1), w1_sf=d(ex.w1_sf), w1_ws2=d(ex.w1_ws2),
                        w2=d(ex.w2), w2_sf=d(ex.w2_sf), w2_ws2=d(ex.w2_ws2))
        self.shared_dev = (d(s.w1[0]), d(s.w1_sf[0]), d(s.w1_ws2), d(s.w2[0]), d(s.w2_sf[0]), d(s.w2_ws2))
        log(f"generated and uploaded {cfg['E']} experts + shared in {time.time() - t0:.1f}s")


def setup_moe(cfg, seed, stack=None):
    import numpy as np
    import torch

    from fp4_block_scaled_route_amd import ops, synth

    if stack is None or stack.key != (cfg["E"], cfg["H"], cfg["I"], seed):
        stack = ExpertStack(cfg, seed)
    x_host = synth.bf16_normal((cfg["T"], cfg["H"]), seed)
    ids, w = synth.route(cfg["T"], cfg["E"], cfg["k"], seed, cfg["routing"])
    mi = synth.MoEInputs(x=x_host, topk_ids=ids, topk_w=w, experts=stack.routed,
                         shared=stack.shared if cfg["shared"] else None)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    dev = dict(topk_ids=d(mi.topk_ids), topk_w=d(mi.topk_w), **stack.dev)
    shared = stack.shared_dev if cfg["shared"] else None
    x = mi.x.cuda()
    t, k, h, i, e = cfg["T"], cfg["k"], cfg["H"], cfg["I"], cfg["E"]
    ws = torch.empty(ops.moe_workspace_size(t, h, i, e, k, shared is not None, cfg["fp4"]),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty((t, h), dtype=torch.bfloat16, device="cuda")
    state = dict(mi=mi, dev=dev, shared=shared, x=x, ws=ws, y=y, stack=stack)
    if cfg["fp4"]:
        # warm-up calibration of the hidden activations' global scale (h kept
        # fp32 for this one call, a2_gs_out = max|h| / 2688)
        xq, xs, gs = ops.quantize_act(x)
        a2 = torch.zeros(1, dtype=torch.float32, device="cuda")
        ws_cal = torch.empty(ops.moe_workspace_size(t, h, i, e, k, shared is not None, False),
                             dtype=torch.uint8, device="cuda")
        ops.moe_grouped(**dev, x_fp4=xq, x_sf=xs, a1_gs=gs, shared=shared, a2_gs_out=a2, workspace=ws_cal, out=y)
        torch.cuda.synchronize()
        del ws_cal
        state.update(xq=xq, xs=xs, gs=gs, a2=a2)
        log(f"calibrated a2_gs = {a2.item():.6g}")
    torch.cuda.synchronize()
    return state


def moe_step(cfg, st, events=None, quantize=True):
    from fp4_block_scaled_route_amd import ops
    if cfg["fp4"]:
        if quantize:
            xq, xs, gs = ops.quantize_act(st["x"], out=(st["xq"], st["xs"]), gs_out=st["gs"])
        else:
            xq, xs, gs = st["xq"], st["xs"], st["gs"]
        return ops.moe_grouped(**st["dev"], x_fp4=xq, x_sf=xs, a1_gs=gs, shared=st["shared"], a2_gs=st["a2"],
                               workspace=st["ws"], out=st["y"], stage_events=events)
    return ops.moe_grouped(**st["dev"], x=st["x"], shared=st["shared"], workspace=st["ws"], out=st["y"],
                           stage_events=events)


SMALL_GROUP_ROWS = 4    # groups with more rows run on the LDS-staged kernel


def moe_accounting(cfg, st, quantize=True):
    """Algorithmic FLOPs and bytes of one step and of the two gate/up GEMM
    launches (groups of > 4 rows, the others), from the routing.  Fully-FP4
    step without the quantizer (quantize=False): the GEMMs read x_fp4 + scales
    instead of bf16 x."""
    import numpy as np
    ids = st["mi"].topk_ids
    e, t, h, i, k = cfg["E"], cfg["T"], cfg["H"], cfg["I"], cfg["k"]
    counts = list(np.bincount(ids.ravel(), minlength=e))
    if cfg["shared"]:
        counts.append(t)
    counts = np.array(counts)
    touched = int((counts[:e] > 0).sum())
    S = 1 if cfg["shared"] else 0
    pairs = t * k + S * t
    flops = pairs * FLOPS_PER_PAIR
    act_in = t * h * 2                                   # bf16 x (the fully-FP4 step quantizes it first)
    if cfg["fp4"]:
        act_in += t * (h // 2 + h // 16) * 2             # x_fp4 + scales written, then read by the GEMM
        if not quantize:
            act_in = t * (h // 2 + h // 16)              # x_fp4 + scales read by the GEMM
    out = t * h * 2
    w_bytes = (touched + S) * (BYTES_PER_EXPERT_W1 + BYTES_PER_EXPERT_W2)
    step_bytes = w_bytes + act_in + out
    row_bytes = (h // 2 + h // 16) if cfg["fp4"] else h * 2   # activation row as the GEMM reads it
    launches = {}
    # more than 16 rows per group on average: one launch of the LDS kernel over all groups
    large_batch = pairs / len(counts) > 16
    big_sel = counts > 0 if large_batch else counts > SMALL_GROUP_ROWS
    for name, sel in (("big", big_sel), ("small", (counts > 0) & ~big_sel)):
        m = counts[sel]
        launches[name] = dict(groups=int(sel.sum()), rows=int(m.sum()),
                              bytes=int(sel.sum()) * BYTES_PER_EXPERT_W1 + int(m.sum()) * row_bytes,
                              flops=int(m.sum()) * 2 * (2 * i * h))
    return dict(touched=touched, flops=flops, step_bytes=step_bytes, g1=launches, large_batch=large_batch)


def moe_cpu_baseline(cfg, st, budget_s=12.0):
    """The oracle, timed on the host on a bounded sample of the same workload:
    consecutive 4-token slices of the batch, each computed in full (all the
    experts its tokens touch), until about budget_s seconds of oracle time."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from fp4_block_scaled_route_amd import synth
    from oracle import moe, quant

    mi = st["mi"]
    shared = mi.shared.expert(0) if mi.shared is not None else None
    a2 = np.float32(st["a2"].item()) if cfg["fp4"] else None
    gs = np.float32(st["gs"].item()) if cfg["fp4"] else None
    total_s, total_bytes, ntok, nexp = 0.0, 0, 0, 0
    for t0 in range(0, cfg["T"], 4):
        toks = list(range(t0, min(cfg["T"], t0 + 4)))
        if cfg["fp4"]:
            rq, rs, rgs = quant.quantize_nvfp4(mi.x[toks].float().numpy(), gs=gs)
            x = np.zeros((cfg["T"], cfg["H"]))
            x[toks] = quant.dequantize_nvfp4(rq, rs, rgs)
        else:
            x = synth.bf16_to_float64(mi.x)
        t_start = time.perf_counter()
        moe.moe_forward(x, mi.topk_ids, mi.topk_w, mi.experts.expert, shared, a2_gs=a2, tokens=toks)
        total_s += time.perf_counter() - t_start
        touched = int(np.unique(mi.topk_ids[toks]).size) + (1 if shared is not None else 0)
        nexp += touched
        total_bytes += touched * (BYTES_PER_EXPERT_W1 + BYTES_PER_EXPERT_W2) + len(toks) * cfg["H"] * 4
        ntok += len(toks)
        if total_s >= budget_s:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return dict(value=round(total_bytes / total_s / 1e9, 4), unit="GB/s", cores=threads, cpu_model=cpu_model(), kind="oracle",
                sample=f"first {ntok} tokens of the batch in 4-token slices ({nexp} expert evaluations), "
                       f"float64 numpy oracle, {total_s:.1f}s of oracle time; elementwise dequantization "
                       f"runs on one thread, matrix products on the BLAS pool",
                seconds=round(total_s, 2))


MOE_NAMES = {"moe_decode": "MoE decode step", "moe_prefill": "MoE prefill chunk",
             "moe_fp4": "fully FP4 MoE at large batch"}


def time_moe(args, cfg, st, quantize=True):
    """Warm-up, then args.steps timed steps: the step time (torch events
    around all steps) and the dominant gate/up launch's time (HIP events the
    library records around that one launch, on its stream)."""
    import torch
    acc = moe_accounting(cfg, st, quantize)
    for _ in range(args.warmup):
        moe_step(cfg, st, quantize=quantize)
    torch.cuda.synchronize()
    hip = HipEvents()
    NEV = 8    # stage i runs from event i to event i + 1
    # dominant kernel: the gate/up launch that streams more weight bytes
    part = "big" if acc["g1"]["big"]["bytes"] > acc["g1"]["small"]["bytes"] else "small"
    k_ev = 1 if part == "big" else 2
    # Timed steps record only the two events around the dominant launch (each
    # recorded event costs a few microseconds between kernels); the per-stage
    # breakdown comes from separate, untimed steps with all eight events.
    kev = [hip.create(2) for _ in range(args.steps)]

    def timed_events(pair):
        ev = [0] * NEV
        ev[k_ev], ev[k_ev + 1] = pair
        return ev

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for s in range(args.steps):
        moe_step(cfg, st, events=timed_events(kev[s]), quantize=quantize)
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / args.steps
    k_list = sorted(hip.elapsed_ms(e[0], e[1]) for e in kev)
    for e in kev:
        hip.destroy(e)
    names = ["permute", "gate_up_big", "gate_up_small", "h_to_f16", "down_big", "down_small", "combine"]
    n_stage_steps = min(args.steps, 5)
    evs = [hip.create(NEV) for _ in range(n_stage_steps)]
    for s in range(n_stage_steps):
        moe_step(cfg, st, events=evs[s], quantize=quantize)
    torch.cuda.synchronize()
    stage = [0.0] * (NEV - 1)
    for s in range(n_stage_steps):
        for i in range(NEV - 1):
            stage[i] += hip.elapsed_ms(evs[s][i], evs[s][i + 1]) / n_stage_steps
    for e in evs:
        hip.destroy(e)
    return dict(acc=acc, part=part, ms_step=ms_step, t_wall=t_wall, k_ms=sum(k_list) / args.steps,
                k_med=k_list[len(k_list) // 2], k_p90=k_list[min(len(k_list) - 1, int(0.9 * len(k_list)))],
                stage={n: round(v, 4) for n, v in zip(names, stage)})


def moe_roofline(args, cfg, tm, src):
    acc, part, k_ms = tm["acc"], tm["part"], tm["k_ms"]
    kern = {"big": "nvfp4_gemm_lds (gate/up + SwiGLU, " +
                   ("all groups: > 16 rows per group on average)" if acc["large_batch"] else "groups of > 4 rows)"),
            "small": "nvfp4_gemm_compact (gate/up + SwiGLU, groups of <= 4 rows)"}[part]
    if cfg["fp4"]:
        kern = kern.replace("nvfp4_gemm_compact", "nvfp4_gemm_direct")
    kb, kf = acc["g1"][part]["bytes"], acc["g1"][part]["flops"]
    traffic = read_traffic(cfg["name"], src)
    if cfg["fp4"]:
        ach = kf / (k_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(ach, 2), peak=FP16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / FP16_PEAK_TFLOPS, 4), traffic=traffic)
    else:
        ach = kb / (k_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(ach / HBM_PEAK_GBS, 4), traffic=traffic)
    roof.update(kernel=kern, kernel_ms=round(k_ms, 4), kernel_ms_median=round(tm["k_med"], 4),
                kernel_ms_p90=round(tm["k_p90"], 4), groups=acc["g1"][part]["groups"],
                algorithmic_bytes_per_launch=kb, algorithmic_flops_per_launch=kf)
    return roof


def run_moe(args, cfg, stack=None, cpu_budget_s=12.0):
    """One MoE workload: the result line (and the state, for reuse)."""
    st = setup_moe(cfg, args.seed, stack)
    src = kernel_source_hash()
    tm = time_moe(args, cfg, st)
    acc, ms_step = tm["acc"], tm["ms_step"]
    gbs = acc["step_bytes"] / (ms_step * 1e-3) / 1e9
    tflops = acc["flops"] / (ms_step * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on a bounded sample of {cfg['name']} ...")
        cpu = moe_cpu_baseline(cfg, st, budget_s=cpu_budget_s)
    result = {
        "metric": "NVFP4 MoE grouped-GEMM TFLOP/s + HBM GB/s (%roofline), 1xMI355X",
        "value": round(tflops, 2) if cfg["fp4"] else round(gbs, 1),
        "unit": "TFLOP/s" if cfg["fp4"] else "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{MOE_NAMES[cfg['name']]}: {cfg['T']} tokens x hidden {cfg['H']}, {cfg['E']} experts "
                               f"top-{cfg['k']} ({cfg['routing']} routing), W1 [4096,7168] W2 [7168,2048] NVFP4"
                               f"{', shared expert' if cfg['shared'] else ''}"
                               f"{', NVFP4 activations (quantizer inside the step)' if cfg['fp4'] else ', bf16 activations'}",
                   "name": cfg["name"], "tokens": cfg["T"], "touched_experts": acc["touched"],
                   "seed": args.seed, "parallelism": "single GPU"},
        "tflops": round(tflops, 2),
        "mfma_frac": round(tflops / FP16_PEAK_TFLOPS, 4),
        "hbm_gbs": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": acc["step_bytes"],
        "algorithmic_flops_per_step": acc["flops"],
        "stage_ms": tm["stage"],
        "stage_note": "per-stage times from separate steps with all stage events recorded",
        "wall_s": round(tm["t_wall"], 4),
        "roofline": moe_roofline(args, cfg, tm, src),
        "cpu_baseline": cpu,
        "kernel_source_hash": src,
    }
    if cfg["fp4"]:
        # the same batch with x already quantized (only nvfp4_moe_grouped timed)
        tq = time_moe(args, cfg, st, quantize=False)
        fl = tq["acc"]["flops"] / (tq["ms_step"] * 1e-3) / 1e12
        result["without_quantize"] = dict(
            ms_per_step=round(tq["ms_step"], 4), tflops=round(fl, 2), mfma_frac=round(fl / FP16_PEAK_TFLOPS, 4),
            hbm_gbs=round(tq["acc"]["step_bytes"] / (tq["ms_step"] * 1e-3) / 1e9, 1),
            roofline=moe_roofline(args, cfg, tq, src), stage_ms=tq["stage"])
    return result, st


def run_headline(args):
    """Default run: the fully-FP4 4096-token batch as the headline line, with
    the decode and prefill steps nested; one expert stack for all three."""
    import torch
    stack = None
    nested = {}
    for name in ("moe_decode", "moe_prefill"):
        res, st = run_moe(args, dict(WORKLOADS[name], name=name), stack, cpu_budget_s=8.0)
        stack = st["stack"]
        for key in ("metric", "n_gpus", "steps", "warmup", "higher_is_better", "scaling", "data",
                    "kernel_source_hash"):
            res.pop(key, None)
        nested[name] = res
        del st
        torch.cuda.synchronize()
    head, _ = run_moe(args, dict(WORKLOADS["moe_fp4"], name="moe_fp4"), stack, cpu_budget_s=8.0)
    head["configs"] = nested
    return head


def time_graph(call, n_calls, reps=5):
    """ms per call of n_calls back-to-back calls captured in one graph and
    replayed reps times: the GPU time of a call with its launches issued
    back to back, without the host work of the Python binding in between
    (which exceeds the GPU time of a microsecond-scale call).  call(i) must
    read the current stream when it runs."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_calls):
            call(i)
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / (reps * n_calls)
    del g
    return ms


def time_eager(call, warmup, steps):
    """ms per call of steps calls issued from Python (host work included)."""
    import torch
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        call(i)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


# ---------------------------------------------------------------------------
# dense linear workload
# ---------------------------------------------------------------------------


def run_linear(args, cfg):
    import numpy as np
    import torch

    from fp4_block_scaled_route_amd import ops, synth

    m, n, k = cfg["M"], cfg["N"], cfg["K"]
    li = synth.make_linear(m, n, k, seed=args.seed)
    w_bytes = n * (k // 2 + k // 16)
    # rotate copies of W so that the working set exceeds the 256 MB last-level cache
    copies = max(1, int(np.ceil(1.0e9 / w_bytes)))
    # the copies are slices of two stacked tensors (no per-copy allocations)
    w_all = torch.from_numpy(li.w).cuda().unsqueeze(0).repeat(copies, 1, 1)
    sf_all = torch.from_numpy(li.w_sf).cuda().unsqueeze(0).repeat(copies, 1, 1)
    ws = [w_all[i] for i in range(copies)]
    sfs = [sf_all[i] for i in range(copies)]
    ws2 = torch.tensor([li.ws2], dtype=torch.float32, device="cuda")
    x = li.x.cuda()
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    need = ops.lib().nvfp4_linear_workspace_size(m, n, k)
    work = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None

    def call(i):
        ops.linear(ws[i % copies], sfs[i % copies], ws2, x=x, out=y, workspace=work)
    ms_eager = time_eager(call, args.warmup, args.steps)
    y_eager = y.clone()
    ms = time_graph(call, args.steps)
    if not torch.equal(y, y_eager):
        raise RuntimeError("graph replay of the linear differs from the eager call")
    # the same calls on one weight copy, which stays in the caches between calls
    ms_warm = time_graph(lambda i: call(0), args.steps)
    nbytes = w_bytes + m * k * 2 + m * n * 2
    flops = 2 * m * n * k
    gbs = nbytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import linear
        log("timing the CPU oracle on a bounded sample ...")
        ms_rows = min(m, 8)
        xs = synth.bf16_to_float64(li.x[:ms_rows])
        t_start = time.perf_counter()
        reps = 0
        while time.perf_counter() - t_start < 10.0:
            linear.linear_bf16(xs, li.w, li.w_sf, li.ws2)
            reps += 1
        sec = (time.perf_counter() - t_start) / reps
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        sample_bytes = w_bytes + ms_rows * k * 2 + ms_rows * n * 2
        cpu = dict(value=round(sample_bytes / sec / 1e9, 4), unit="GB/s", cores=threads, cpu_model=cpu_model(), kind="oracle",
                   sample=f"{ms_rows} token row{'s' if ms_rows > 1 else ''} against the whole weight, float64 numpy oracle, {reps} "
                          f"repetitions in about 10 s; dequantization runs on one thread, the product on the "
                          f"BLAS pool")
    return {
        "metric": "NVFP4 linear HBM GB/s (%roofline), 1xMI355X", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"dense NVFP4 linear x[{m},{k}] @ W[{n},{k}]^T, bf16 out, {copies} rotating "
                               f"weight copies", "name": args.workload,
                   "timing": f"{args.steps} back-to-back calls captured in one graph, replayed 5 times"},
        "eager_ms_per_call": round(ms_eager, 5), "workspace_bytes": need,
        "cache_warm_ms_per_call": round(ms_warm, 5),
        "cache_warm_note": "one weight copy reused by every call (cached between calls); not the headline figure",
        "tflops": round(flops / (ms * 1e-3) / 1e12, 3), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None),
        "cpu_baseline": cpu,
    }


def run_router(args, cfg):
    """Router gate: logits of T tokens against the FP8 round-tripped weight,
    then top-k softmax (one nvfp4_router_topk call: the logits GEMM and the
    selection)."""
    import numpy as np
    import torch

    from fp4_block_scaled_route_amd import ops, synth

    t, h, e, k = cfg["T"], cfg["H"], cfg["E"], cfg["k"]
    x = synth.bf16_normal((t, h), args.seed).cuda()
    w = synth.router_weight(e, h, args.seed)
    w_bytes = e * h * 2
    copies = max(1, int(np.ceil(1.0e9 / w_bytes)))   # rotate weights past the last-level cache
    w_rt, _ = ops.router_prepare(w.cuda())
    wrs = [w_rt.clone() for _ in range(copies)]
    logits = torch.empty((t, e), dtype=torch.float32, device="cuda")
    ids = torch.empty((t, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((t, k), dtype=torch.float32, device="cuda")
    work = torch.empty(max(1, ops.router_workspace_size(t, h, e)), dtype=torch.uint8, device="cuda")
    def call(i):
        ops.router_topk(x, wrs[i % copies], k, logits, ids, wts, work)
    ms_eager = time_eager(call, args.warmup, args.steps)
    ms = time_graph(call, args.steps)
    # algorithmic: weight + activations read, logits written, selection written
    nbytes = w_bytes + t * h * 2 + t * e * 4 + t * k * 8
    flops = 2 * t * e * h
    gbs = nbytes / (ms * 1e-3) / 1e9
    tfl = flops / (ms * 1e-3) / 1e12
    bound_mfma = flops / nbytes > BF16_RIDGE_FLOP_PER_BYTE
    if bound_mfma:
        roof = dict(bound="mfma", achieved=round(tfl, 2), peak=FP16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(tfl / FP16_PEAK_TFLOPS, 4), traffic=None)
    else:
        roof = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None)
    roof.update(kernel="nvfp4_router_logits + nvfp4_router_select (one call)", kernel_ms=round(ms, 5),
                algorithmic_bytes_per_launch=nbytes, algorithmic_flops_per_launch=flops)
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import router
        log("timing the CPU oracle on a bounded sample ...")
        _, _, wr_ref = router.router_weight_roundtrip(w.float().numpy())
        xs = synth.bf16_to_float64(x[:16].cpu())
        t_start = time.perf_counter()
        reps = 0
        while time.perf_counter() - t_start < 10.0:
            router.route(xs, wr_ref, k)
            reps += 1
        sec = (time.perf_counter() - t_start) / reps
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        sample_bytes = w_bytes + 16 * h * 2 + 16 * e * 4 + 16 * k * 8
        cpu = dict(value=round(sample_bytes / sec / 1e9, 4), unit="GB/s", cores=threads, cpu_model=cpu_model(), kind="oracle",
                   sample=f"16 tokens against the whole weight, float64 numpy oracle, {reps} repetitions in "
                          f"about 10 s")
    return {
        "metric": "router gate GB/s or TFLOP/s (%roofline), 1xMI355X",
        "value": round(gbs if not bound_mfma else tfl, 3), "unit": "GB/s" if not bound_mfma else "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"router gate: {t} tokens x hidden {h}, {e} experts, top-{k} softmax, FP8 "
                               f"round-tripped bf16 weight, {copies} rotating weight copies",
                   "name": args.workload,
                   "timing": f"{args.steps} back-to-back calls captured in one graph, replayed 5 times"},
        "eager_ms_per_call": round(ms_eager, 5),
        "tflops": round(tfl, 3), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": roof, "cpu_baseline": cpu,
    }


def run_grouped_linear(args, cfg):
    """Grouped linear of the attention output projection (wo_a): x [T, G, K]
    bf16 times G NVFP4 weights [N, K] (one nvfp4_grouped_linear call, the
    fp16 staging of x included)."""
    import numpy as np
    import torch

    from fp4_block_scaled_route_amd import ops, synth

    t, g, n, k = cfg["T"], cfg["G"], cfg["N"], cfg["K"]
    gi = synth.make_grouped_linear(t, g, n, k, seed=args.seed)
    x = gi.x.cuda()
    w_bytes = g * n * (k // 2 + k // 16)
    copies = max(1, int(np.ceil(1.0e9 / (w_bytes + t * g * k * 2))))   # rotate past the last-level cache
    ws = [(torch.from_numpy(gi.w).cuda(), torch.from_numpy(gi.w_sf).cuda()) for _ in range(min(copies, 64))]
    ws2 = torch.from_numpy(gi.ws2).cuda()
    xs = [x.clone() for _ in range(min(copies, 8))]
    y = torch.empty((t, g, n), dtype=torch.bfloat16, device="cuda")
    need = ops.grouped_linear_workspace_size(t, g, n, k)
    work = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    nw, nx = len(ws), len(xs)

    def call(i):
        ops.grouped_linear(*ws[i % nw], ws2, x=xs[i % nx], out=y, workspace=work)
    ms_eager = time_eager(call, args.warmup, args.steps)
    ms = time_graph(call, args.steps)
    nbytes = w_bytes + t * g * k * 2 + t * g * n * 2
    flops = 2 * t * g * n * k
    gbs = nbytes / (ms * 1e-3) / 1e9
    tfl = flops / (ms * 1e-3) / 1e12
    bound_mfma = flops / nbytes > BF16_RIDGE_FLOP_PER_BYTE
    if bound_mfma:
        roof = dict(bound="mfma", achieved=round(tfl, 2), peak=FP16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(tfl / FP16_PEAK_TFLOPS, 4), traffic=None)
    else:
        roof = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None)
    roof.update(kernel="grouped GEMM (one call: one launch up to 4 tokens, else fp16 staging + GEMM)",
                kernel_ms=round(ms, 5),
                algorithmic_bytes_per_launch=nbytes, algorithmic_flops_per_launch=flops)
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import grouped_linear
        log("timing the CPU oracle on a bounded sample ...")
        xs64 = synth.bf16_to_float64(gi.x[:4])
        t_start = time.perf_counter()
        reps = 0
        while time.perf_counter() - t_start < 10.0:
            grouped_linear.grouped_linear_bf16(xs64, gi.w, gi.w_sf, gi.ws2)
            reps += 1
        sec = (time.perf_counter() - t_start) / reps
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        sample_bytes = w_bytes + 4 * g * k * 2 + 4 * g * n * 2
        cpu = dict(value=round(sample_bytes / sec / 1e9, 4), unit="GB/s", cores=threads, cpu_model=cpu_model(), kind="oracle",
                   sample=f"4 tokens against all {g} group weights, float64 numpy oracle, {reps} repetitions "
                          f"in about 10 s")
    return {
        "metric": "wo_a grouped linear GB/s or TFLOP/s (%roofline), 1xMI355X",
        "value": round(gbs if not bound_mfma else tfl, 3), "unit": "GB/s" if not bound_mfma else "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"grouped linear wo_a: {t} tokens x {g} groups, K {k} per group, width {n}, "
                               f"NVFP4 weights, bf16 activations, {nw} rotating weight copies",
                   "name": args.workload,
                   "timing": f"{args.steps} back-to-back calls captured in one graph, replayed 5 times"},
        "eager_ms_per_call": round(ms_eager, 5),
        "tflops": round(tfl, 3), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": roof, "cpu_baseline": cpu,
    }


def run_rmsnorm_quant(args, cfg):
    """RMSNorm fused with the NVFP4 quantizer (one nvfp4_rmsnorm_quantize call,
    global scale computed), timed beside the unfused path it must equal: the
    RMSNorm pass writing bf16 y, then nvfp4_quantize_act on y."""
    import torch

    from fp4_block_scaled_route_amd import ops, synth

    t, k = cfg["T"], cfg["K"]
    eps = 1e-6
    copies = max(1, min(16, int(1.0e9 // (t * k * 2))))   # rotate inputs past the last-level cache
    xs = [synth.bf16_normal((t, k), args.seed + i).cuda() for i in range(copies)]
    w = (synth.bf16_normal((k,), args.seed + 999).float() * 0.5 + 1.0).to(torch.bfloat16).cuda()
    q = torch.empty((t, k // 2), dtype=torch.uint8, device="cuda")
    sf = torch.empty((t, k // 16), dtype=torch.uint8, device="cuda")
    gs = torch.zeros(1, dtype=torch.float32, device="cuda")
    y = torch.empty((t, k), dtype=torch.bfloat16, device="cuda")
    work = torch.empty(max(16, ops.lib().nvfp4_rmsnorm_quantize_workspace_size(t)), dtype=torch.uint8, device="cuda")
    L = ops.lib()
    qwork = torch.empty(max(16, L.nvfp4_quantize_act_workspace_size(t, k)), dtype=torch.uint8, device="cuda")

    def fused(i):
        s = torch.cuda.current_stream().cuda_stream
        ops._check(L.nvfp4_rmsnorm_quantize(xs[i % copies].data_ptr(), w.data_ptr(), eps, t, k, None,
                                            gs.data_ptr(), 1, q.data_ptr(), sf.data_ptr(), work.data_ptr(),
                                            work.numel(), s))

    def unfused(i):
        s = torch.cuda.current_stream().cuda_stream
        ops._check(L.nvfp4_rmsnorm_quantize(xs[i % copies].data_ptr(), w.data_ptr(), eps, t, k, y.data_ptr(),
                                            gs.data_ptr(), 1, q.data_ptr(), sf.data_ptr(), work.data_ptr(),
                                            work.numel(), s))
        ops._check(L.nvfp4_quantize_act(y.data_ptr(), t, k, gs.data_ptr(), 1, q.data_ptr(), sf.data_ptr(),
                                        qwork.data_ptr(), qwork.numel(), s))

    ms_eager = time_eager(fused, args.warmup, args.steps)
    ms = time_graph(fused, args.steps)
    time_eager(unfused, args.warmup, 1)
    ms_unfused = time_graph(unfused, args.steps)
    nbytes = t * k * 2 + k * 2 + t * (k // 2) + t * (k // 16) + 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import rmsnorm
        log("timing the CPU oracle on a bounded sample ...")
        rows = min(t, 64)
        xh = xs[0][:rows].float().cpu().numpy()
        wh = w.float().cpu().numpy()
        t_start = time.perf_counter()
        reps = 0
        while time.perf_counter() - t_start < 10.0:
            rmsnorm.rmsnorm_quantize(xh, wh, eps)
            reps += 1
        sec = (time.perf_counter() - t_start) / reps
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        sample_bytes = rows * k * 2 + k * 2 + rows * (k // 2) + rows * (k // 16) + 4
        cpu = dict(value=round(sample_bytes / sec / 1e9, 4), unit="GB/s", cores=threads, cpu_model=cpu_model(), kind="oracle",
                   sample=f"{rows} rows of {k}, float32/float64 numpy oracle, {reps} repetitions in about 10 s")
    return {
        "metric": "RMSNorm + NVFP4 quantization GB/s (%roofline), 1xMI355X",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"RMSNorm of x [{t}, {k}] bf16 with a bf16 weight, fused with the NVFP4 quantizer "
                               f"(global scale computed), {copies} rotating inputs", "name": args.workload,
                   "timing": f"{args.steps} back-to-back calls captured in one graph, replayed 5 times"},
        "eager_ms_per_call": round(ms_eager, 5), "unfused_ms": round(ms_unfused, 5),
        "roofline": dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None,
                         kernel="nvfp4_rmsnorm_stats + nvfp4_rmsnorm_quant (one call)", kernel_ms=round(ms, 5),
                         algorithmic_bytes_per_launch=nbytes),
        "cpu_baseline": cpu,
    }


def run_copy(args):
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE /
    WRITE_SIZE readings to bytes."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n, "launches": 3}))


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="headline", choices=["headline"] + sorted(WORKLOADS),
                    help="headline (default): the fully-FP4 4096-token batch with the decode and prefill "
                         "steps nested; or one workload")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this path has no multi-GPU "
              "mode. It would shard by experts for prefill (each GPU owns E/G experts; token rows go "
              "all-to-all before and after the grouped GEMMs) and over the intermediate size for decode "
              "(each GPU streams 1/G of every touched expert; y is reduced)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be >= 1 and --warmup >= 0")
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        run_copy(args)
        return
    if args.workload == "headline":
        res = run_headline(args)
    else:
        cfg = dict(WORKLOADS[args.workload], name=args.workload)
        if cfg["kind"] == "moe":
            res, _ = run_moe(args, cfg)
        else:
            run = {"linear": run_linear, "router": run_router,
                   "grouped_linear": run_grouped_linear, "rmsnorm_quant": run_rmsnorm_quant}[cfg["kind"]]
            res = run(args, cfg)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
