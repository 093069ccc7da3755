"""Empty batches (no tokens) through the MoE layer, the router and the fused
RMSNorm + quantization, through the C ABI: the other sizes are still
checked, no output row exists to be written, and a quantizer asked to compute
the activation global scale writes 0, the amax of no elements.  (The dense
and grouped linear and the plain quantizer have their own empty-input
tests.)"""
import numpy as np
import pytest
import torch

from gpu_util import DeviceExperts, dev, f32, say
from fp4_block_scaled_route_amd import ops, synth

pytestmark = pytest.mark.gpu


def _moe_inputs():
    mi = synth.make_moe(4, 256, 256, 8, 2, seed=1, shared=True)
    return mi, DeviceExperts(mi.experts), DeviceExperts(mi.shared)


def test_moe_zero_tokens():
    say("moe T=0 (bf16 and NVFP4 activations)")
    mi, de, ds = _moe_inputs()
    ids, w = dev(mi.topk_ids[:0]), dev(mi.topk_w[:0])
    off = torch.full((8 + 2,), -7, dtype=torch.int32, device="cuda")
    y = ops.moe_grouped(ids, w, **de.args(), x=dev(mi.x[:0]), shared=ds.as_shared(), offsets_out=off)
    y4 = ops.moe_grouped(ids, w, **de.args(), x_fp4=torch.empty((0, 128), dtype=torch.uint8, device="cuda"),
                         x_sf=torch.empty((0, 16), dtype=torch.uint8, device="cuda"), a1_gs=f32(0.01),
                         a2_gs=f32(0.5), shared=ds.as_shared())
    torch.cuda.synchronize()
    assert y.shape == (0, 256) and y4.shape == (0, 256)
    assert (off.cpu().numpy() == -7).all(), "offsets written for an empty batch"


def test_moe_zero_tokens_still_checks_shapes():
    """The library's own size check at T = 0, called through the C ABI (the
    binding would reject the inconsistent tensors before the call)."""
    mi, de, ds = _moe_inputs()
    a = ops.MoeArgs()
    a.T, a.H, a.I, a.E, a.topk = 0, 200, 256, 8, 2     # hidden 200: not a multiple of 256
    a.x = de.w1.data_ptr()
    a.topk_ids, a.topk_w = de.w1.data_ptr(), de.w1.data_ptr()
    a.w1, a.w1_sf, a.w1_ws2 = de.w1.data_ptr(), de.w1_sf.data_ptr(), de.w1_ws2.data_ptr()
    a.w2, a.w2_sf, a.w2_ws2 = de.w2.data_ptr(), de.w2_sf.data_ptr(), de.w2_ws2.data_ptr()
    a.y = de.w1.data_ptr()
    ws = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    import ctypes
    assert ops.lib().nvfp4_moe_grouped(ctypes.byref(a), None) == -2


def test_router_zero_tokens():
    say("router T=0")
    w_rt, _ = ops.router_prepare(dev(synth.router_weight(16, 256, seed=2)))
    x = dev(synth.bf16_normal((1, 256), 3)[:0])
    logits, ids, wts = ops.router_topk(x, w_rt, 4)
    torch.cuda.synchronize()
    assert logits.shape == (0, 16) and ids.shape == (0, 4) and wts.shape == (0, 4)
    with pytest.raises(ops.Nvfp4Error) as e:
        ops.router_topk(x, w_rt, 17)      # top-17 of 16 experts
    assert e.value.status == -2


def test_quantizers_zero_rows_write_gs():
    say("quantize / rmsnorm+quantize T=0")
    x = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(512, dtype=torch.bfloat16, device="cuda")
    g1, g2, given = f32(7.0), f32(7.0), f32(3.0)
    q, sf, g = ops.rmsnorm_quantize(x, w, 1e-6, gs_out=g1)
    q2, sf2, _ = ops.rmsnorm_quantize(x, w, 1e-6, gs=given)
    _, _, g3 = ops.quantize_act(x, gs_out=g2)
    torch.cuda.synchronize()
    assert q.shape == (0, 256) and sf.shape == (0, 32) and q2.shape == (0, 256) and sf2.shape == (0, 32)
    assert g.item() == 0.0 and g3.item() == 0.0, "computed gs of no elements"
    assert given.item() == 3.0, "a supplied gs is input only"
    with pytest.raises(ops.Nvfp4Error) as e:
        ops.rmsnorm_quantize(x, w, 0.0)
    assert e.value.status == -6


def test_rmsnorm_gs_out_is_overwritten():
    """A caller's gs buffer holding a stale value: the computed gs replaces
    it (it is reset on the device, not accumulated into)."""
    x = synth.bf16_normal((3, 256), 5)
    w = torch.ones(256, dtype=torch.bfloat16)
    stale = f32(1e6)
    _, _, g = ops.rmsnorm_quantize(x.cuda(), w.cuda(), 1e-6, gs_out=stale)
    _, _, ref = ops.rmsnorm_quantize(x.cuda(), w.cuda(), 1e-6)
    torch.cuda.synchronize()
    assert g.item() == ref.item() and np.isfinite(g.item()) and 0 < g.item() < 1e6
