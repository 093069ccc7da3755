"""CPU checks of the Python binding's argument validation: every tensor's
dtype, shape, contiguity and device is checked before its pointer reaches
the C ABI (which cannot see any of them).  Tensors here live on the CPU, so a
call whose arguments are all consistent stops at the device check; every
other case must stop earlier, at its own mismatch.  No library call is made."""
import pytest
import torch

from fp4_block_scaled_route_amd import ops

T, H, I, E, K = 3, 256, 256, 4, 2


def _moe(**over):
    a = dict(topk_ids=torch.zeros((T, K), dtype=torch.int32), topk_w=torch.zeros((T, K)),
             w1=torch.zeros((E, 2 * I, H // 2), dtype=torch.uint8),
             w1_sf=torch.zeros((E, 2 * I, H // 16), dtype=torch.uint8), w1_ws2=torch.zeros(E),
             w2=torch.zeros((E, H, I // 2), dtype=torch.uint8),
             w2_sf=torch.zeros((E, H, I // 16), dtype=torch.uint8), w2_ws2=torch.zeros(E),
             x=torch.zeros((T, H), dtype=torch.bfloat16))
    a.update(over)
    return a


def _shared(**over):
    s = dict(s1=torch.zeros((2 * I, H // 2), dtype=torch.uint8), s1_sf=torch.zeros((2 * I, H // 16), dtype=torch.uint8),
             s1_ws2=torch.zeros(1), s2=torch.zeros((H, I // 2), dtype=torch.uint8),
             s2_sf=torch.zeros((H, I // 16), dtype=torch.uint8), s2_ws2=torch.zeros(1))
    s.update(over)
    return tuple(s.values())


def _raises(fn, exc, text, **kw):
    with pytest.raises(exc) as e:
        fn(**kw)
    assert text in str(e.value), str(e.value)


def test_moe_consistent_cpu_tensors_stop_at_the_device_check():
    _raises(ops.moe_grouped, ValueError, "must be on the GPU", **_moe())
    _raises(ops.moe_grouped, ValueError, "must be on the GPU", **_moe(shared=_shared()))


@pytest.mark.parametrize("over,exc,text", [
    (dict(topk_ids=torch.zeros((T, K), dtype=torch.int64)), TypeError, "call .int()"),
    (dict(topk_w=torch.zeros((T, K), dtype=torch.float64)), TypeError, "topk_w has dtype"),
    (dict(topk_w=torch.zeros((T, K + 1))), ValueError, "topk_w has shape"),
    (dict(x=torch.zeros((T - 1, H), dtype=torch.bfloat16)), ValueError, "x has shape"),
    (dict(x=torch.zeros((T, H), dtype=torch.float16)), TypeError, "x has dtype"),
    (dict(x=torch.zeros((H, T), dtype=torch.bfloat16).t()), ValueError, "x must be contiguous"),
    (dict(out=torch.zeros((T, H - 16), dtype=torch.bfloat16)), ValueError, "out has shape"),
    (dict(w1_ws2=torch.zeros(E - 1)), ValueError, "w1_ws2 has shape"),
    (dict(w2=torch.zeros((E, H, I), dtype=torch.uint8)), ValueError, "w2 has shape"),
    (dict(w2_sf=torch.zeros((E, I // 16, H), dtype=torch.uint8)), ValueError, "w2_sf has shape"),
    (dict(w1=torch.zeros((E, 2 * I + 1, H // 2), dtype=torch.uint8)), ValueError, "even count"),
    (dict(x_fp4=torch.zeros((T, H // 2), dtype=torch.uint8)), ValueError, "pass either x or"),
    (dict(x=None), ValueError, "pass either x or"),
    (dict(x=None, x_fp4=torch.zeros((T, H // 2), dtype=torch.uint8), x_sf=torch.zeros((T, H // 16), dtype=torch.uint8)),
     ValueError, "need all of"),
    (dict(a2_gs=torch.zeros(2)), ValueError, "a2_gs must hold exactly one element"),
    (dict(offsets_out=torch.zeros(E + 1, dtype=torch.int32)), ValueError, "offsets_out has shape"),
    (dict(perm_out=torch.zeros(T * K, dtype=torch.int32)), ValueError, "perm_out has shape"),
    (dict(workspace=torch.zeros(16, dtype=torch.int32)), TypeError, "workspace has dtype"),
    (dict(shared=_shared(s2=torch.zeros((H, I), dtype=torch.uint8))), ValueError, "s2) has shape"),
    (dict(shared=_shared(s1_ws2=torch.zeros(2))), ValueError, "s1_ws2) must hold exactly one"),
    (dict(shared=_shared()[:5]), ValueError, "shared must be"),
])
def test_moe_mismatches(over, exc, text):
    _raises(ops.moe_grouped, exc, text, **_moe(**over))


def test_moe_mixed_devices_are_reported():
    if not hasattr(torch, "device"):
        pytest.skip()
    meta = torch.zeros((T, H), dtype=torch.bfloat16, device="meta")
    _raises(ops.moe_grouped, ValueError, "on the GPU", **_moe(x=meta))


def _lin(**over):
    a = dict(w=torch.zeros((64, 128), dtype=torch.uint8), w_sf=torch.zeros((64, 16), dtype=torch.uint8),
             ws2=torch.zeros(1), x=torch.zeros((5, 256), dtype=torch.bfloat16))
    a.update(over)
    return a


@pytest.mark.parametrize("over,exc,text", [
    ({}, ValueError, "must be on the GPU"),
    (dict(x=torch.zeros((5, 512), dtype=torch.bfloat16)), ValueError, "x has shape"),
    (dict(w_sf=torch.zeros((64, 8), dtype=torch.uint8)), ValueError, "w_sf has shape"),
    (dict(ws2=torch.zeros(1, dtype=torch.float64)), TypeError, "ws2 has dtype"),
    (dict(out=torch.zeros((5, 32), dtype=torch.bfloat16)), ValueError, "out has shape"),
    (dict(gsa=torch.zeros(1)), ValueError, "pass either x or"),
    (dict(x=None, x_fp4=torch.zeros((5, 128), dtype=torch.uint8), x_sf=torch.zeros((5, 16), dtype=torch.uint8),
          gsa=torch.zeros(1), out=torch.zeros((5, 64), dtype=torch.float32)), TypeError, "out has dtype"),
])
def test_linear_mismatches(over, exc, text):
    _raises(ops.linear, exc, text, **_lin(**over))


def _glin(**over):
    a = dict(w=torch.zeros((8, 32, 128), dtype=torch.uint8), w_sf=torch.zeros((8, 32, 16), dtype=torch.uint8),
             ws2=torch.zeros(8), x=torch.zeros((2, 8, 256), dtype=torch.bfloat16))
    a.update(over)
    return a


@pytest.mark.parametrize("over,exc,text", [
    ({}, ValueError, "must be on the GPU"),
    (dict(ws2=torch.zeros(1)), ValueError, "ws2 has shape"),
    (dict(x=torch.zeros((2, 4, 256), dtype=torch.bfloat16)), ValueError, "x has shape"),
    (dict(x=torch.zeros((2, 8 * 256), dtype=torch.bfloat16)), ValueError, "must be 3-D"),
])
def test_grouped_linear_mismatches(over, exc, text):
    _raises(ops.grouped_linear, exc, text, **_glin(**over))


def test_quantizer_and_rmsnorm_mismatches():
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    _raises(ops.quantize_act, ValueError, "must be on the GPU", x=x)
    _raises(ops.quantize_act, TypeError, "x has dtype", x=x.float())
    _raises(ops.quantize_act, ValueError, "out[1] has shape",
            x=x, out=(torch.zeros((4, 128), dtype=torch.uint8), torch.zeros((4, 8), dtype=torch.uint8)))
    _raises(ops.quantize_act, ValueError, "gs must hold exactly one", x=x, gs=torch.zeros(2))
    w = torch.ones(256, dtype=torch.bfloat16)
    _raises(ops.rmsnorm_quantize, ValueError, "must be on the GPU", x=x, w=w, eps=1e-6)
    _raises(ops.rmsnorm_quantize, ValueError, "w has shape", x=x, w=w[:128], eps=1e-6)
    _raises(ops.rmsnorm_quantize, ValueError, "y has shape", x=x, w=w, eps=1e-6,
            y=torch.zeros((3, 256), dtype=torch.bfloat16))


def test_router_mismatches():
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    w = torch.zeros((16, 256), dtype=torch.bfloat16)
    _raises(ops.router_prepare, ValueError, "must be on the GPU", w=w)
    _raises(ops.router_prepare, TypeError, "w has dtype", w=w.float())
    _raises(ops.router_topk, ValueError, "must be on the GPU", x=x, w_rt=w, topk=4)
    _raises(ops.router_topk, ValueError, "w_rt has shape", x=x, w_rt=w[:, :128], topk=4)
    _raises(ops.router_topk, TypeError, "ids has dtype", x=x, w_rt=w, topk=4,
            ids=torch.zeros((4, 4), dtype=torch.int64))
