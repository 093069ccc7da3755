"""The no-allocation MoE entry point (nvfp4_moe_grouped_noalloc) through the
C ABI: its output equals nvfp4_moe_grouped's (with a caller workspace) bit
for bit on consecutive calls that share the library's static scratch array,
the second with a smaller batch, and it stays within the oracle's tolerance
and per-element bound."""
import numpy as np
import pytest
import torch

from gpu_util import DeviceExperts, calibrate_a2, compare, dev, f32, say
from fp4_block_scaled_route_amd import ops, synth
from moe_bound import check_elementwise, reference_and_bound
from oracle import quant

pytestmark = pytest.mark.gpu


def _both(de, ds, ids, w, **kw):
    t = ids.shape[0]
    h = de.w1.shape[2] * 2
    y_ws = ops.moe_grouped(dev(ids), dev(w), **de.args(), shared=ds.as_shared() if ds else None, **kw)
    y_na = torch.full((t, h), float("nan"), dtype=torch.bfloat16, device="cuda")
    ops.moe_grouped(dev(ids), dev(w), **de.args(), shared=ds.as_shared() if ds else None, out=y_na,
                    noalloc=True, **kw)
    torch.cuda.synchronize()
    return y_ws, y_na


def test_noalloc_matches_workspace_entry_two_calls():
    # 24 tokens, hidden 4096, 128 experts, top-8 + shared: under 2 rows per
    # group, so the gate/up K split (partial sums and counters in the
    # scratch array) is active; then 5 tokens on the same array
    t, h, i, e, k = 24, 4096, 512, 128, 8
    say(f"noalloc: T={t} H={h} I={i} E={e} k={k} shared, then T=5")
    mi = synth.make_moe(t, h, i, e, k, seed=41, shared=True, threads=8)
    assert (t * k + t) / (e + 1) <= 2.0
    de, ds = DeviceExperts(mi.experts), DeviceExperts(mi.shared)
    y_ws, y_na = _both(de, ds, mi.topk_ids, mi.topk_w, x=dev(mi.x))
    assert torch.equal(y_ws, y_na), "noalloc output differs from the workspace entry point"
    x64 = synth.bf16_to_float64(mi.x)
    ref, bound, _ = reference_and_bound(x64, mi.topk_ids, mi.topk_w, mi.experts, mi.shared, workers=8)
    compare(y_na, ref, what="noalloc T=24")
    check_elementwise(y_na.float().cpu().numpy(), ref, bound, what="noalloc T=24")
    # second call, smaller batch, same scratch array
    t2 = 5
    y_ws2, y_na2 = _both(de, ds, mi.topk_ids[:t2], mi.topk_w[:t2], x=dev(mi.x[:t2]))
    assert torch.equal(y_ws2, y_na2), "second (smaller) noalloc call differs"
    assert torch.equal(y_na2, y_na[:t2]), "a token's output depends on the batch it is in"


def test_noalloc_fully_fp4_and_capacity():
    t, h, i, e, k = 16, 1024, 512, 16, 4
    say(f"noalloc fully fp4: T={t} H={h} I={i} E={e} k={k}")
    mi = synth.make_moe(t, h, i, e, k, seed=42, shared=False, threads=4)
    de = DeviceExperts(mi.experts)
    xq, xs, gs = ops.quantize_act(dev(mi.x))
    rq, rs, rgs = quant.quantize_nvfp4(mi.x.float().numpy())
    xa = quant.dequantize_nvfp4(rq, rs, rgs)
    a2 = calibrate_a2(xa, mi.topk_ids, mi.experts, range(t))
    y_ws, y_na = _both(de, None, mi.topk_ids, mi.topk_w, x_fp4=xq, x_sf=xs, a1_gs=gs, a2_gs=f32(a2))
    assert torch.equal(y_ws, y_na)
    y_ws2, y_na2 = _both(de, None, mi.topk_ids[:3], mi.topk_w[:3], x_fp4=xq[:3], x_sf=xs[:3], a1_gs=gs,
                         a2_gs=f32(a2))
    assert torch.equal(y_ws2, y_na2)
    # a batch beyond the scratch array is refused on the host, nothing launched
    big_t = 4096
    ids = torch.zeros((big_t, k), dtype=torch.int32, device="cuda")
    wts = torch.zeros((big_t, k), dtype=torch.float32, device="cuda")
    x = torch.zeros((big_t, h), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((big_t, h), dtype=torch.bfloat16, device="cuda")
    # (hidden 1024: even 4096 tokens may fit; use the DeepSeek sizes' limit instead)
    need = ops.moe_workspace_size(big_t, h, i, e, k, False, False)
    if need > (72 << 20):
        with pytest.raises(ops.Nvfp4Error) as err:
            ops.moe_grouped(ids, wts, **de.args(), x=x, out=out, noalloc=True)
        assert err.value.status == -7
