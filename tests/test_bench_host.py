"""Host logic of bench.py: the algorithmic byte and FLOP accounting of the MoE
workloads on hand-built routings (group counts, the split of the gate/up
GEMM into launches, bytes per step), checked against sums worked out by
hand from the layer's sizes, and the one-GPU rule of the command line."""
import os
import subprocess
import sys
import types

import numpy as np

import bench

H, I = 7168, 2048
W1 = 2 * I * (H // 2) + 2 * I * (H // 16)     # gate/up codes 14,680,064 + scales 1,835,008
W2 = H * (I // 2) + H * (I // 16)             # down codes 7,340,032 + scales 917,504


def _acc(ids, **over):
    cfg = dict(bench.WORKLOADS["moe_decode"], **over)
    return bench.moe_accounting(cfg, {"mi": types.SimpleNamespace(topk_ids=np.array(ids, dtype=np.int32))})


def test_per_expert_constants():
    assert W1 == 16_515_072 and W2 == 8_257_536
    assert bench.BYTES_PER_EXPERT_W1 == W1 and bench.BYTES_PER_EXPERT_W2 == W2
    assert W1 + W2 == 24_772_608
    # one (token, expert) pair: a [1, H] x [H, 2I] and a [1, I] x [I, H] product, 2 FLOPs per term
    assert bench.FLOPS_PER_PAIR == 2 * (H * 2 * I) + 2 * (I * H) == 88_080_384


def test_small_batch_accounting():
    # 4 tokens, top-2 of 8 experts: expert 0 gets 3 rows, 1 and 2 get 2, 3 gets 1; shared expert 4 rows
    a = _acc([[0, 1], [0, 2], [3, 0], [1, 2]], T=4, E=8, k=2)
    assert a["touched"] == 4 and not a["large_batch"]
    assert a["flops"] == 12 * bench.FLOPS_PER_PAIR                      # 8 routed + 4 shared pairs
    assert a["step_bytes"] == 5 * (W1 + W2) + 4 * H * 2 + 4 * H * 2       # weights + bf16 x in + y out
    # no group has more than 4 rows: every group in the small-group launch
    assert a["g1"]["big"]["groups"] == 0
    assert a["g1"]["small"] == dict(groups=5, rows=12, bytes=5 * W1 + 12 * H * 2, flops=12 * 2 * 2 * I * H)


def test_big_groups_split_off():
    # 8 tokens, top-1: expert 5 gets 6 rows (> 4), expert 2 gets 2; no shared expert
    a = _acc([[5]] * 6 + [[2]] * 2, T=8, E=8, k=1, shared=False)
    assert a["touched"] == 2 and not a["large_batch"]
    assert a["g1"]["big"] == dict(groups=1, rows=6, bytes=W1 + 6 * H * 2, flops=6 * 4 * I * H)
    assert a["g1"]["small"] == dict(groups=1, rows=2, bytes=W1 + 2 * H * 2, flops=2 * 4 * I * H)


def test_large_batch_and_fp4_rows():
    # 64 tokens, top-2 of 4 experts + shared: 192 pairs over 5 groups (> 16 rows per group):
    # one launch over all groups, NVFP4 activation rows (codes + scale bytes)
    ids = [[t % 4, (t + 1) % 4] for t in range(64)]
    a = _acc(ids, T=64, E=4, k=2, fp4=True)
    row = H // 2 + H // 16
    assert a["large_batch"] and a["g1"]["small"]["groups"] == 0
    assert a["g1"]["big"] == dict(groups=5, rows=192, bytes=5 * W1 + 192 * row, flops=192 * 4 * I * H)
    # x read, its NVFP4 copy written and read again, y written
    assert a["step_bytes"] == 5 * (W1 + W2) + 64 * H * 2 + 64 * row * 2 + 64 * H * 2


def test_more_than_one_gpu_is_refused():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
