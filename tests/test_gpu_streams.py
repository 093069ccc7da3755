"""nvfp4_moe_grouped on a non-default stream and captured into a HIP graph.

The result must not depend on the stream the call is made on; the call must
be capturable into a graph and give the same result on every replay, with
eager work between the replays; the stage events are recorded in order.  The
eager result of the small case is checked against the oracle, the stream and
graph runs bit for bit against the eager result (the arithmetic of every
output row is fixed by the routing and the inputs); the large-batch path's
parity with the oracle is the MoE parity tests' part, here its replays are
compared with its eager call."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import DeviceExperts, compare, dev, say
from fp4_block_scaled_route_amd import ops, synth
from oracle import moe

pytestmark = pytest.mark.gpu

# 148 (token, expert) pairs over 16 experts (about 9 rows a group, so both
# GEMM launches, groups of > 4 rows and the others, have work), shared expert
T, H, I, E, K = 37, 512, 256, 16, 4


def _setup():
    mi = synth.make_moe(T, H, I, E, K, seed=21, routing="zipf", shared=True, threads=2)
    de, ds = DeviceExperts(mi.experts), DeviceExperts(mi.shared)
    ws = torch.empty(ops.moe_workspace_size(T, H, I, E, K, True, False), dtype=torch.uint8, device="cuda")
    args = dict(topk_ids=dev(mi.topk_ids), topk_w=dev(mi.topk_w), **de.args(), x=dev(mi.x),
                shared=ds.as_shared(), workspace=ws)
    ref = moe.moe_forward(synth.bf16_to_float64(mi.x), mi.topk_ids, mi.topk_w, mi.experts.expert,
                          mi.shared.expert(0), tokens=None)
    counts = np.bincount(mi.topk_ids.ravel(), minlength=E)
    assert (counts > 4).any() and ((counts > 0) & (counts <= 4)).any()
    return args, ref


def test_moe_side_stream_matches_default_stream():
    say("moe on a non-default stream")
    args, ref = _setup()
    y0 = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ops.moe_grouped(**args, out=y0)
    torch.cuda.synchronize()
    compare(y0, ref, what="default stream")
    s = torch.cuda.Stream()
    y1 = torch.zeros_like(y0)
    with torch.cuda.stream(s):
        ops.moe_grouped(**args, out=y1)
    s.synchronize()
    assert torch.equal(y0, y1)


def test_moe_graph_capture_and_replay():
    say("moe captured into a graph, replayed three times")
    args, ref = _setup()
    y0 = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ops.moe_grouped(**args, out=y0)
    torch.cuda.synchronize()
    compare(y0, ref, what="eager")
    s = torch.cuda.Stream()
    yg = torch.zeros_like(y0)
    with torch.cuda.stream(s):              # warm-up on the capture stream
        ops.moe_grouped(**args, out=yg)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ops.moe_grouped(**args, out=yg)
    torch.cuda.synchronize()
    ws2 = torch.empty_like(args["workspace"])
    other = torch.empty_like(y0)
    for rep in range(3):
        yg.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y0), f"replay {rep} differs from the eager result"
        # eager work between replays, on its own workspace
        ops.moe_grouped(**{**args, "workspace": ws2}, out=other)
        torch.cuda.synchronize()
        assert torch.equal(other, y0)


def test_moe_stage_events_in_order():
    say("moe stage events")
    args, _ = _setup()
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(8):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ops.moe_grouped(**args, out=y, stage_events=evs)
    torch.cuda.synchronize()
    ms = ctypes.c_float()
    for i in range(7):
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(evs[i]),
                                       ctypes.c_void_p(evs[i + 1])) == 0
        assert ms.value >= 0.0, (i, ms.value)
    # NULL entries are skipped: only the pair around the first gate/up launch
    y2 = torch.empty_like(y)
    ops.moe_grouped(**args, out=y2, stage_events=[0, evs[1], evs[2], 0, 0, 0, 0, 0])
    torch.cuda.synchronize()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(evs[1]), ctypes.c_void_p(evs[2])) == 0
    assert ms.value >= 0.0
    assert torch.equal(y, y2)
    for e in evs:
        hip.hipEventDestroy(ctypes.c_void_p(e))


def test_moe_fully_fp4_large_batch_graph_replay():
    """The large-batch path (every group on the eight-wave kernel, NVFP4
    activations and NVFP4 h, groups of more than one 112-row pass) captured
    into a graph: every replay equals the eager call bit for bit."""
    t, h, i, e, k = 600, 1024, 1024, 16, 4       # 150 rows a group on average, shared expert 600 rows
    say(f"fully-FP4 large batch captured into a graph T={t} H={h} I={i} E={e} k={k}")
    mi = synth.make_moe(t, h, i, e, k, seed=23, routing="uniform", shared=True, threads=2)
    de, ds = DeviceExperts(mi.experts), DeviceExperts(mi.shared)
    xq, xs, gs = ops.quantize_act(dev(mi.x))
    ids, w = dev(mi.topk_ids), dev(mi.topk_w)
    # the hidden activations' global scale from the fp32-h path of the same call
    a2 = torch.zeros(1, dtype=torch.float32, device="cuda")
    ops.moe_grouped(ids, w, **de.args(), x_fp4=xq, x_sf=xs, a1_gs=gs, shared=ds.as_shared(), a2_gs_out=a2)
    torch.cuda.synchronize()
    assert float(a2.item()) > 0.0
    ws = torch.empty(ops.moe_workspace_size(t, h, i, e, k, True, True), dtype=torch.uint8, device="cuda")
    args = dict(topk_ids=ids, topk_w=w, **de.args(), x_fp4=xq, x_sf=xs, a1_gs=gs, shared=ds.as_shared(),
                a2_gs=a2, workspace=ws)
    y0 = torch.empty((t, h), dtype=torch.bfloat16, device="cuda")
    ops.moe_grouped(**args, out=y0)
    torch.cuda.synchronize()
    assert torch.isfinite(y0.float()).all() and y0.float().abs().max() > 0
    s = torch.cuda.Stream()
    yg = torch.zeros_like(y0)
    with torch.cuda.stream(s):
        ops.moe_grouped(**args, out=yg)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ops.moe_grouped(**args, out=yg)
    torch.cuda.synchronize()
    ws2 = torch.empty_like(ws)
    other = torch.empty_like(y0)
    for rep in range(3):
        yg.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y0), f"replay {rep} differs from the eager result"
        ops.moe_grouped(**{**args, "workspace": ws2}, out=other)
        torch.cuda.synchronize()
        assert torch.equal(other, y0)
