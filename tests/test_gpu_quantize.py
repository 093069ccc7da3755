"""GPU parity of nvfp4_quantize_act: codes, scale bytes and the global scale
must equal the oracle's bit for bit (the quantizer is an integer decision
taken in float32 on both sides)."""
import numpy as np
import pytest
import torch

from gpu_util import dev, f32, say
from fp4_block_scaled_route_amd import ops, synth
from oracle import quant

pytestmark = pytest.mark.gpu


def _inputs(kind, m, k, seed):
    if kind == "normal":
        return synth.bf16_normal((m, k), seed)
    rng = np.random.default_rng(seed)
    if kind == "wide":          # rows spanning many binades, zero blocks, ties
        x = rng.standard_normal((m, k)) * np.exp(rng.uniform(-20, 20, (m, 1)))
        x[:, 16:32] = 0.0
        x[0, :16] = [0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, -6]
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    if kind == "zeros":
        return torch.zeros((m, k), dtype=torch.bfloat16)
    raise ValueError(kind)


@pytest.mark.parametrize("kind,m,k", [("normal", 64, 7168), ("normal", 3, 48), ("wide", 37, 512),
                                      ("zeros", 4, 256), ("normal", 4096, 7168)])
def test_quantize_bit_exact(kind, m, k):
    say(f"quantize {kind} [{m},{k}]")
    x = _inputs(kind, m, k, seed=11)
    q, sf, gs = ops.quantize_act(dev(x))
    torch.cuda.synchronize()
    rq, rs, rgs = quant.quantize_nvfp4(x.float().numpy())
    assert gs.item() == float(rgs)
    assert np.array_equal(sf.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("gs_value", [0.001, 1.0, 0.0])
def test_quantize_supplied_gs(gs_value):
    say(f"quantize supplied gs {gs_value}")
    x = _inputs("normal", 16, 1024, seed=3)
    gs = f32(gs_value)
    q, sf, gs_out = ops.quantize_act(dev(x), gs=gs)
    torch.cuda.synchronize()
    rq, rs, _ = quant.quantize_nvfp4(x.float().numpy(), gs=np.float32(gs_value))
    assert gs_out.item() == np.float32(gs_value)
    assert np.array_equal(sf.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


def test_quantize_empty():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    q, sf, gs = ops.quantize_act(x)
    torch.cuda.synchronize()
    assert q.shape == (0, 128) and gs.item() == 0.0
