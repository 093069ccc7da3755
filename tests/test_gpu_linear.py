"""GPU parity of nvfp4_linear against the float64 oracle."""
import numpy as np
import pytest
import torch

from gpu_util import compare, dev, f32, say
from fp4_block_scaled_route_amd import ops, synth
from moe_bound import check_elementwise, linear_reference_and_bound
from oracle import linear, quant

pytestmark = pytest.mark.gpu


def _run_bf16(li):
    return ops.linear(dev(li.w), dev(li.w_sf), f32(li.ws2), x=dev(li.x))


@pytest.mark.parametrize("m,n,k", [
    (8, 128, 256),                                      # single NVFP4 linear, seed 0
    (1, 1536, 7168), (32, 1536, 7168), (128, 1536, 7168),   # projection shape
    (1, 24576, 1536), (32, 24576, 1536), (128, 24576, 1536),
    (17, 48, 512), (100, 64, 256), (129, 32, 768),      # ragged token counts (several passes)
    (3, 96, 2304), (2, 64, 8448),                       # bf16 staging: 8 loads per lane (partly masked);
                                                        # rows longer than 8192 (read twice)
])
def test_linear_bf16(m, n, k):
    say(f"linear bf16 M={m} N={n} K={k}")
    li = synth.make_linear(m, n, k, seed=0)
    y = _run_bf16(li)
    torch.cuda.synchronize()
    ref, bound = linear_reference_and_bound(synth.bf16_to_float64(li.x), li.w, li.w_sf, li.ws2)
    compare(y, ref, what=f"linear {m}x{n}x{k}")
    check_elementwise(y.float().cpu().numpy(), ref, bound, what=f"linear {m}x{n}x{k}")


def test_linear_hand_worked_golden():
    from conftest import golden_dict
    g = golden_dict("linear_example.txt")
    # the fixture has K=16; pad K to 256 with zero codes (K must be a multiple of 256)
    w = np.zeros((16, 128), np.uint8)
    sf = np.zeros((16, 16), np.uint8)
    w[0, :8] = [int(b, 16) for b in g["w_row0"]]
    w[1, :8] = [int(b, 16) for b in g["w_row1"]]
    sf[0, 0] = int(g["sf"][0], 16)
    sf[1, 0] = int(g["sf"][1], 16)
    x = np.zeros((2, 256), np.float32)
    x[0, :16] = [float(v) for v in g["x_row0"]]
    x[1, :16] = [float(v) for v in g["x_row1"]]
    y = ops.linear(dev(w), dev(sf), f32(float(g["ws2"][0])), x=dev(torch.from_numpy(x).to(torch.bfloat16)))
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    assert y[0, 0] == 12 and y[0, 1] == -13 and y[1, 0] == -0.5 and y[1, 1] == -1.375
    assert not y[:, 2:].any()


def test_linear_extreme_activation_range():
    """bf16 activations far outside fp16's range are staged exactly (per-row
    power-of-two shift)."""
    li = synth.make_linear(4, 64, 512, seed=2)
    x = li.x.float()
    x[0] *= 2.0 ** 100
    x[1] *= 2.0 ** -100
    x[2, :] = 0
    li.x = x.to(torch.bfloat16)
    y = _run_bf16(li)
    torch.cuda.synchronize()
    ref = linear.linear_bf16(synth.bf16_to_float64(li.x), li.w, li.w_sf, li.ws2)
    for r in (0, 1, 3):
        compare(y[r:r + 1], ref[r:r + 1], what=f"row {r}")
    assert not y[2].float().abs().sum()


@pytest.mark.parametrize("m,k", [(4, 1536), (1, 7168)])
def test_linear_wide_binade_spread_within_a_row(m, k):
    """Rows whose magnitudes span more than 29 binades: the fp16 staging
    shifts each row (each 256-element chunk of it, at most 4 rows) so its
    maximum lands in [2^14, 2^15), so elements more than 29 binades below
    that maximum fall on fp16 subnormals (or flush to zero below 2^-24 after
    the shift).  Each output element stays within its
    bound, which carries 2^-39 * max|x_row| * sum_k |W[n, k]| for that
    rounding besides the accumulation and output roundings."""
    say(f"linear binade spread M={m} K={k}")
    li = synth.make_linear(m, 256, k, seed=5)
    x = li.x.float()
    rng = np.random.default_rng(5)
    for r in range(m):
        # per element a power of two between 2^-34 and 2^6: a 40-binade spread
        x[r] *= torch.from_numpy(np.exp2(rng.integers(-34, 7, size=k)).astype(np.float32))
    li.x = x.to(torch.bfloat16)
    xr = synth.bf16_to_float64(li.x)
    mx = np.abs(xr).max(axis=1)
    tiny = np.abs(xr) < mx[:, None] * 2.0 ** -29
    assert tiny.sum(axis=1).min() > k // 10, "rows must hold elements below the exact staging range"
    y = _run_bf16(li)
    torch.cuda.synchronize()
    ref, bound = linear_reference_and_bound(xr, li.w, li.w_sf, li.ws2)
    compare(y, ref, what=f"binade spread {m}x{k}")
    check_elementwise(y.float().cpu().numpy(), ref, bound, what=f"binade spread {m}x{k}")


@pytest.mark.parametrize("m,n,k", [
    (1, 1536, 7168), (4, 1536, 7168),      # projection shape: K split over the waves of a workgroup
    (2, 24576, 1536),                      # wide projection: 6 chunks streamed by one wave
    (3, 1552, 7424),                       # 29 chunks (last range shorter); 97 fragments (last tile half)
    (4, 64, 8448),                         # 33 chunks
    (4, 48, 256), (1, 16, 256),            # one chunk; one fragment
])
def test_linear_small_m_one_launch(m, n, k):
    """At most 4 rows: one launch with no workspace (activations converted in
    LDS per chunk; K up to 8 chunks streamed by one wave, longer K split over
    the waves of a workgroup and added in LDS), bf16 and NVFP4 activations,
    every element within its bound."""
    say(f"linear one launch M={m} N={n} K={k}")
    assert ops.lib().nvfp4_linear_workspace_size(m, n, k) == 0
    li = synth.make_linear(m, n, k, seed=6)
    w, sf, g2 = dev(li.w), dev(li.w_sf), f32(li.ws2)
    y = ops.linear(w, sf, g2, x=dev(li.x))
    xq, xs, gs = ops.quantize_act(dev(li.x))
    y4 = ops.linear(w, sf, g2, x_fp4=xq, x_sf=xs, gsa=gs)
    torch.cuda.synchronize()
    ref, bound = linear_reference_and_bound(synth.bf16_to_float64(li.x), li.w, li.w_sf, li.ws2)
    compare(y, ref, what=f"one launch {m}x{n}x{k}")
    check_elementwise(y.float().cpu().numpy(), ref, bound, what=f"one launch {m}x{n}x{k}")
    rq, rs, rgs = quant.quantize_nvfp4(li.x.float().numpy())
    assert np.array_equal(xq.cpu().numpy(), rq) and np.array_equal(xs.cpu().numpy(), rs)
    ref4 = linear.linear_nvfp4(rq, rs, rgs, li.w, li.w_sf, li.ws2)
    _, bound4 = linear_reference_and_bound(quant.dequantize_nvfp4(rq, rs, rgs), li.w, li.w_sf, li.ws2, x_fp4=True)
    compare(y4, ref4, what=f"one launch NVFP4 {m}x{n}x{k}")
    check_elementwise(y4.float().cpu().numpy(), ref4, bound4, what=f"one launch NVFP4 {m}x{n}x{k}")


def test_linear_four_rows_long_k_takes_the_staged_path():
    """4 rows of K = 16384: 16 waves of 4-chunk ranges would need more LDS
    than a workgroup has, so the call takes the staged path (fp16 copy in the
    workspace, barrier-free kernel with a K split)."""
    m, n, k = 4, 64, 16384
    assert ops.lib().nvfp4_linear_workspace_size(m, n, k) > 0
    say(f"linear staged path M={m} N={n} K={k}")
    li = synth.make_linear(m, n, k, seed=7)
    y = _run_bf16(li)
    torch.cuda.synchronize()
    ref, bound = linear_reference_and_bound(synth.bf16_to_float64(li.x), li.w, li.w_sf, li.ws2)
    check_elementwise(y.float().cpu().numpy(), ref, bound, what="staged 4x64x16384")


def test_linear_workspace_reused_across_shapes_and_graph_replays():
    """One workspace serves a sequence of calls of different shapes (the
    one-launch calls need none), and a captured graph of one-launch calls
    replays correctly several times, with eager work in between."""
    say("linear workspace reuse and graph replays")
    n, k = 1536, 7168
    need = max(ops.lib().nvfp4_linear_workspace_size(mm, n, k) for mm in (1, 4, 32))
    work = torch.empty(need, dtype=torch.uint8, device="cuda")
    li = synth.make_linear(32, n, k, seed=8)
    w, sf, g2 = dev(li.w), dev(li.w_sf), f32(li.ws2)
    x = dev(li.x)
    ref, bound = linear_reference_and_bound(synth.bf16_to_float64(li.x), li.w, li.w_sf, li.ws2)
    for mm in (32, 1, 4, 32, 2):
        y = ops.linear(w, sf, g2, x=x[:mm], workspace=work)
        torch.cuda.synchronize()
        check_elementwise(y.float().cpu().numpy(), ref[:mm], bound[:mm], what=f"reuse M={mm}")
    y_eager = ops.linear(w, sf, g2, x=x[:1])
    out = torch.empty_like(y_eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ops.linear(w, sf, g2, x=x[:1], out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(3):
            ops.linear(w, sf, g2, x=x[:1], out=out)
    for rep in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, y_eager), f"replay {rep}"
        ops.linear(w, sf, g2, x=x[:4], workspace=work)   # eager work between the replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("m,n,k", [(8, 128, 256), (128, 1536, 7168), (33, 256, 1536)])
def test_linear_nvfp4_activations(m, n, k):
    say(f"linear nvfp4 M={m} N={n} K={k}")
    li = synth.make_linear(m, n, k, seed=1)
    xq, xs, gs = ops.quantize_act(dev(li.x))
    y = ops.linear(dev(li.w), dev(li.w_sf), f32(li.ws2), x_fp4=xq, x_sf=xs, gsa=gs)
    torch.cuda.synchronize()
    rq, rs, rgs = quant.quantize_nvfp4(li.x.float().numpy())
    ref = linear.linear_nvfp4(rq, rs, rgs, li.w, li.w_sf, li.ws2)
    compare(y, ref, what="nvfp4 x nvfp4")
    _, bound = linear_reference_and_bound(quant.dequantize_nvfp4(rq, rs, rgs), li.w, li.w_sf, li.ws2, x_fp4=True)
    check_elementwise(y.float().cpu().numpy(), ref, bound, what="nvfp4 x nvfp4")


def test_linear_empty_and_errors():
    li = synth.make_linear(1, 16, 256, seed=0)
    y = ops.linear(dev(li.w), dev(li.w_sf), f32(li.ws2), x=dev(li.x[:0]))
    assert y.shape == (0, 16)
    with pytest.raises(ops.Nvfp4Error) as e:
        ops.linear(dev(li.w[:, :100]), dev(li.w_sf[:, :12]), f32(li.ws2), x=dev(li.x[:, :200]))
    assert e.value.status == -2


@pytest.mark.parametrize("m,n,k", [(1, 1536, 7168), (32, 1536, 7168)])
def test_linear_split_k_is_deterministic(m, n, k):
    """K is split over waves (one-launch kernel at M = 1) or work items
    (four-wave kernel at M = 32); the partial sums are added in a fixed
    order, so repeated calls agree bit for bit."""
    say(f"linear K split determinism M={m}")
    li = synth.make_linear(m, n, k, seed=4)
    y1 = _run_bf16(li)
    y2 = _run_bf16(li)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
