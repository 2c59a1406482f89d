"""Pins of the oracle's codecs against the format tables and an independent library decoder."""
import json
import math
import os

import numpy as np
import torch

import oracle
from oracle import brute


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "e2m1_e4m3_values.json")) as f:
        return json.load(f)


def test_e2m1_all_codes_match_table(golden_dir):
    g = _golden(golden_dir)["e2m1"]
    for c in range(16):
        v = oracle.e2m1(c)
        assert v == g[str(c)]
        assert math.copysign(1.0, v) == math.copysign(1.0, g[str(c)])  # code 8 is -0
        assert v == float(brute.e2m1(c))


def test_e4m3_all_bytes_match_torch_float8():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        v = oracle.e4m3fn(b)
        if np.isnan(ref[b]):
            assert math.isnan(v), hex(b)
        else:
            assert v == ref[b], hex(b)
            assert math.copysign(1.0, v) == math.copysign(1.0, ref[b])
            assert v == float(brute.e4m3(b))


def test_e4m3_anchor_values(golden_dir):
    for k, want in _golden(golden_dir)["e4m3_anchors"].items():
        v = oracle.e4m3fn(int(k, 16))
        if want == "nan":
            assert math.isnan(v)
        else:
            assert v == want and math.copysign(1, v) == math.copysign(1, want), k


def test_hand_worked_products(golden_dir):
    for case in _golden(golden_dir)["hand_worked_products"]:
        v = oracle.e2m1(int(case["e2m1"], 16)) * oracle.e4m3fn(int(case["e4m3"], 16))
        assert v == case["value"]


def test_bf16_matches_torch():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F80, 0xFF80, 0x0001, 0x7F7F, 0x4049, 0x3E80],
                    dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for b, r in zip(bits, ref):
        assert oracle.bf16(int(b)) == r
    assert math.isnan(oracle.bf16(0x7FC1))


def test_decode_matrix_matches_brute():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, size=(3, 32), dtype=np.uint8)
    scales = rng.integers(0, 0x7E, size=(3, 2), dtype=np.uint8)
    W = oracle.decode_matrix(codes, scales)
    for n in range(3):
        for k in range(64):
            assert W[n, k] == float(brute.weight(codes, scales, n, k))
