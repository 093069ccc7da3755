"""Pins of the oracle's number formats against the format specification,
hand-worked examples and torch's own float8_e4m3fn conversion."""
import math

import numpy as np
import pytest
import torch

from conftest import golden_dict, read_golden
from oracle import codec


def test_e2m1_table_matches_spec():
    for code, val in read_golden("e2m1_values.txt"):
        want = float(val)
        got = codec.E2M1_VALUES[int(code)]
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)


def test_e4m3_spot_values_match_spec():
    for b, val in read_golden("e4m3_spot_values.txt"):
        got = codec.E4M3_VALUES[int(b, 16)]
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), b


def test_e4m3_decode_matches_torch_for_all_bytes():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = codec.E4M3_VALUES
    both_nan = np.isnan(lib) & np.isnan(ours)
    assert np.all(both_nan | (lib == ours))


def test_e4m3_encode_round_trip_every_finite_byte():
    b = np.arange(0x7F, dtype=np.uint8)          # non-negative finite bytes
    assert np.array_equal(codec.e4m3fn_encode_nonneg(codec.E4M3_VALUES[b]), b)


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(0, 464, 200000), rng.uniform(0, 0.02, 100000),
                        np.exp(rng.uniform(-12, 6.1, 100000))]).astype(np.float32)
    v = v[v <= 464.0]
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codec.e4m3fn_encode_nonneg(v), lib)
    # midpoints between neighbouring values: ties go to the even byte
    vals = codec.E4M3_VALUES[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2
    enc = codec.e4m3fn_encode_nonneg(mids)
    lib = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(enc, lib)
    assert np.all(enc % 2 == 0)


def test_e4m3_encode_saturates():
    assert list(codec.e4m3fn_encode_nonneg(np.array([448.0, 464.0, 500.0, 1e30]))) == [0x7E] * 4


def test_e2m1_rne_ties():
    for v, code in read_golden("e2m1_rne_ties.txt"):
        got = int(codec.e2m1_encode(np.array([float(v)], dtype=np.float32))[0])
        assert got == int(code), (v, got, code)


def test_e2m1_encode_decode_round_trip():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(codec.e2m1_encode(codec.E2M1_VALUES[codes]), codes)


def test_pack_unpack_nibble_order():
    # element 2j is the low nibble
    assert list(codec.unpack_fp4(np.array([0xA7], np.uint8))) == [0x7, 0xA]
    rng = np.random.default_rng(0)
    p = rng.integers(0, 256, (5, 24), dtype=np.uint8)
    assert np.array_equal(codec.pack_fp4(codec.unpack_fp4(p)), p)


def test_dequant_hand_worked_examples():
    ws2 = np.float32(0.002)
    for b, s, e0, e1 in read_golden("dequant_examples.txt"):
        packed = np.full((1, 8), int(b, 16), np.uint8)     # 16 elements = 1 block
        sf = np.array([[int(s, 16)]], np.uint8)
        d = codec.dequant_nvfp4(packed, sf, 1.0)
        assert d[0, 0] == float(e0) and d[0, 1] == float(e1), (b, d[0, :2])
        assert np.all(d[0, 0::2] == float(e0)) and np.all(d[0, 1::2] == float(e1))
        d2 = codec.dequant_nvfp4(packed, sf, ws2)
        assert d2[0, 0] == float(e0) * float(ws2)


def test_lut_times_scale_is_exact_in_fp16_and_bf16():
    """Every E2M1 x E4M3 product (finite scales) has <= 5 significant bits and
    lies in [2^-10, 2688]: exact in fp16 and in bf16 (the GPU decode relies on it)."""
    prod = np.outer(codec.E2M1_VALUES, codec.E4M3_VALUES[:0x7F]).ravel()
    assert np.array_equal(prod.astype(np.float16).astype(np.float64), prod)
    t = torch.from_numpy(prod)
    assert torch.equal(t.to(torch.bfloat16).to(torch.float64), t)
    nz = np.abs(prod[prod != 0])
    assert nz.min() == 2.0 ** -10 and nz.max() == 2688.0
