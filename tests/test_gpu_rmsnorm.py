"""GPU parity of nvfp4_rmsnorm_quantize (RMSNorm fused with the NVFP4
quantizer) against the oracle, through the C ABI: the RMSNorm output, the
codes, the scale bytes and the global scale are compared bit for bit, and the
fused result equals the unfused path (the quantizer run on the RMSNorm
output) bit for bit."""
import numpy as np
import pytest
import torch

from gpu_util import compare, dev, say
from fp4_block_scaled_route_amd import ops, synth
from oracle import linear, rmsnorm

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _inputs(t, k, seed):
    x = synth.bf16_normal((t, k), seed)
    w = (synth.bf16_normal((k,), seed + 1000).float() * 0.5 + 1.0).to(torch.bfloat16)
    return x, w


def _check(t, k, seed, x=None, w=None):
    if x is None:
        x, w = _inputs(t, k, seed)
    y = torch.empty((t, k), dtype=torch.bfloat16, device="cuda")
    q, sf, gs = ops.rmsnorm_quantize(x.cuda(), w.cuda(), EPS, y=y)
    torch.cuda.synchronize()
    ry, rq, rs, rg = rmsnorm.rmsnorm_quantize(x.float().numpy(), w.float().numpy(), EPS)
    assert np.array_equal(y.float().cpu().numpy(), ry), "RMSNorm output"
    assert gs.item() == float(rg)
    assert np.array_equal(sf.cpu().numpy(), rs) and np.array_equal(q.cpu().numpy(), rq)
    return x, w, y, q, sf, gs


@pytest.mark.parametrize("t,k", [(1, 256), (37, 1536), (64, 7168), (300, 7168), (5, 10240)])
def test_rmsnorm_quantize_bit_exact(t, k):
    say(f"rmsnorm+quantize T={t} K={k}")
    _check(t, k, seed=t)


def test_rmsnorm_quantize_full_batch_bit_exact():
    say("rmsnorm+quantize 4096 x 7168")
    _check(4096, 7168, seed=3)


def test_fused_equals_unfused_on_the_gpu():
    """The pages' A/B check: the quantizer on the RMSNorm output gives the
    same global scale, codes and scale bytes as the fused call."""
    say("rmsnorm fused vs unfused")
    x, w, y, q, sf, gs = _check(64, 7168, seed=5)
    q2, sf2, gs2 = ops.quantize_act(y)
    torch.cuda.synchronize()
    assert gs2.item() == gs.item() and torch.equal(q2, q) and torch.equal(sf2, sf)


def test_supplied_global_scale_and_edge_rows():
    say("rmsnorm supplied gs, zero and extreme rows")
    x, w = _inputs(8, 512, seed=6)
    xf = x.float()
    xf[1] = 0.0
    xf[2] *= 2.0 ** 100
    xf[3] *= 2.0 ** -100
    x = xf.to(torch.bfloat16)
    _check(8, 512, seed=0, x=x, w=w)
    gsv = torch.tensor([0.0007], dtype=torch.float32, device="cuda")
    q, sf, _ = ops.rmsnorm_quantize(x.cuda(), w.cuda(), EPS, gs=gsv)
    torch.cuda.synchronize()
    _, rq, rs, _ = rmsnorm.rmsnorm_quantize(x.float().numpy(), w.float().numpy(), EPS, gs=np.float32(0.0007))
    assert np.array_equal(q.cpu().numpy(), rq) and np.array_equal(sf.cpu().numpy(), rs)


def test_feeds_the_linear():
    """RMSNorm + quantization feeding the q_a projection (NVFP4 activations)."""
    say("rmsnorm+quantize -> linear q_a")
    x, w = _inputs(16, 7168, seed=7)
    li = synth.make_linear(16, 1536, 7168, seed=8)
    q, sf, gs = ops.rmsnorm_quantize(x.cuda(), w.cuda(), EPS)
    ylin = ops.linear(dev(li.w), dev(li.w_sf), torch.tensor([li.ws2], dtype=torch.float32, device="cuda"),
                      x_fp4=q, x_sf=sf, gsa=gs)
    torch.cuda.synchronize()
    _, rq, rs, rg = rmsnorm.rmsnorm_quantize(x.float().numpy(), w.float().numpy(), EPS)
    ref = linear.linear_nvfp4(rq, rs, float(rg), li.w, li.w_sf, li.ws2)
    compare(ylin, ref, what="rmsnorm -> linear")


def test_wide_spread_rows_r_within_one_ulp():
    """Rows whose squares span far more than fp64's 53 bits: the fp64 sums of
    squares are then inexact, and the kernel's summation order (four partial
    sums per lane, then across lanes) and the oracle's (numpy's pairwise sum)
    may differ in the last bit.  r stays within one fp32 ulp of the oracle's
    (the workspace's first T floats hold r per row), and y is bit-exact in
    every row where r is."""
    t, k = 64, 7168
    say(f"rmsnorm wide-spread rows T={t} K={k}")
    rng = np.random.default_rng(11)
    x = synth.bf16_normal((t, k), 11).float()
    x *= torch.from_numpy(np.exp2(rng.integers(-60, 11, size=(t, k))).astype(np.float32))
    x = x.to(torch.bfloat16)
    _, w = _inputs(1, k, seed=12)
    xs = x.float().numpy().astype(np.float64) ** 2
    spread = xs.max(axis=1) / np.where(xs > 0, xs, np.inf).min(axis=1)
    assert (spread > 2.0 ** 100).all(), "rows must span more than the exact fp64 sum range"
    work = torch.empty(ops.lib().nvfp4_rmsnorm_quantize_workspace_size(t), dtype=torch.uint8, device="cuda")
    y = torch.empty((t, k), dtype=torch.bfloat16, device="cuda")
    q, sf, gs = ops.rmsnorm_quantize(x.cuda(), w.cuda(), EPS, y=y, workspace=work)
    torch.cuda.synchronize()
    r_gpu = work[:4 * t].view(torch.float32).cpu().numpy()
    r_ref = rmsnorm.rms_scale(x.float().numpy(), EPS)
    assert np.all(np.abs(r_gpu.astype(np.float64) - r_ref) <= np.abs(np.spacing(r_ref))), "r within one ulp"
    eq = r_gpu == r_ref
    ry = rmsnorm.rmsnorm_bf16(x.float().numpy(), w.float().numpy(), EPS)
    assert np.array_equal(y.float().cpu().numpy()[eq], ry[eq])
    say(f"  rows with r equal to the oracle's: {int(eq.sum())} of {t}")
    if eq.all():
        _, rq, rs, rg = rmsnorm.rmsnorm_quantize(x.float().numpy(), w.float().numpy(), EPS)
        assert gs.item() == float(rg)
        assert np.array_equal(q.cpu().numpy(), rq) and np.array_equal(sf.cpu().numpy(), rs)
