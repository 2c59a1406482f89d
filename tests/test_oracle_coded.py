"""Pins of the oracle's coded-activation path (or_e8m0, or_dequant_coded, or_layer_coded).

Reading (the pages name gate/up over E4M3-coded activations but give no
activation scale): activations are E4M3FN codes with one E8M0 scale per 32,
x = e4m3(code) * 2^(scale - 127). Pinned against exact fractions built from the
bit fields independently of the oracle (oracle/brute.py), torch's float8
decode, and a hand-worked example; the layer against the bf16 layer on the same
values and against exact rational brute force on a tiny layer.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import brute


def test_e8m0_is_a_power_of_two_and_ff_is_nan():
    for b in range(255):
        assert oracle.e8m0(b) == float(Fraction(2) ** (b - 127)), b
    assert math.isnan(oracle.e8m0(255))
    if hasattr(torch, "float8_e8m0fnu"):
        t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
        for b in range(255):
            assert oracle.e8m0(b) == t[b], b


def test_dequant_every_code_at_several_scales():
    codes = np.arange(256, dtype=np.uint8)
    t8 = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for sb in (0, 1, 100, 120, 127, 128, 140, 200, 254):
        x = oracle.dequant_coded(np.tile(codes, 1).reshape(8, 32), np.full((8, 1), sb, dtype=np.uint8)).reshape(-1)
        for c in range(256):
            v = brute.e4m3(c)
            if v is None:
                assert math.isnan(x[c]) and math.isnan(t8[c])
            else:
                want = v * Fraction(2) ** (sb - 127)
                assert x[c] == float(want), (c, sb)           # exact
                assert x[c] == t8[c] * 2.0 ** (sb - 127), (c, sb)


def test_dequant_hand_worked_and_group_mapping():
    # 0x38 = 1.0, 0x40 = 2.0, 0xC4 = -3.0, 0x01 = 2^-9; scales 2^1 for k < 32, 2^-3 for k >= 32
    codes = np.zeros((1, 64), dtype=np.uint8)
    codes[0, [0, 1, 31, 32, 63]] = [0x38, 0x40, 0xC4, 0x01, 0x38]
    scales = np.array([[128, 124]], dtype=np.uint8)
    x = oracle.dequant_coded(codes, scales)[0]
    assert x[0] == 2.0 and x[1] == 4.0 and x[31] == -6.0
    assert x[32] == 2.0 ** -12 and x[63] == 0.125
    assert np.count_nonzero(x) == 5
    bad = scales.copy()
    bad[0, 1] = 255
    y = oracle.dequant_coded(codes, bad)[0]
    assert np.all(np.isnan(y[32:])) and not np.any(np.isnan(y[:32]))


def test_coded_layer_equals_bf16_layer_on_the_same_values():
    cfg = synth.CONFIGS["tiny"]
    ex = {e: synth.layer_expert(cfg, 0, e) for e in range(cfg.E)}
    codes, scales = synth.coded_activations(cfg.seed, 0, cfg.R, cfg.H)
    _, lg = synth.layer_inputs(cfg, 0)
    xf = oracle.dequant_coded(codes, scales)
    xb = synth.f32_to_bf16_bits(xf.astype(np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(xb).astype(np.float64), xf)   # every value is a bf16 value
    a = oracle.layer_coded(codes, scales, lg, ex, cfg.H, cfg.I, cfg.E, cfg.k)
    b = oracle.layer(xb, lg, ex, cfg.H, cfg.I, cfg.E, cfg.k)
    for n in ("topk_id", "topk_w", "act", "out", "y"):
        assert np.array_equal(a[n], b[n]), n


def test_coded_layer_gate_up_against_exact_fractions():
    """H 64, I 32, E 3, top-2, two rows: act from the exact rational g and u
    (SwiGLU evaluated in float64 on the correctly rounded g, u) within a few ulps."""
    H, I, E, k, R = 64, 32, 3, 2, 2
    ex = {e: synth.expert(77, 0, e, H, I, -2, 1) for e in range(E)}
    codes, scales = synth.coded_activations(78, 0, R, H, -9, -6)
    lg = synth.logits(78, 0, R, E)
    res = oracle.layer_coded(codes, scales, lg, ex, H, I, E, k)
    for r in range(R):
        xq = []
        for i in range(H):
            v = brute.e4m3(int(codes[r, i]))
            xq.append(v * Fraction(2) ** (int(scales[r, i // 32]) - 127))
        for j in range(k):
            e = ex[int(res["topk_id"][r, j])]
            g = brute.matvec(e["gate_codes"], e["gate_scales"], xq)
            u = brute.matvec(e["up_codes"], e["up_scales"], xq)
            for n in range(I):
                gf, uf = float(g[n]), float(u[n])
                ex_ = math.exp(-gf) if -gf < 709.0 else math.inf   # exp overflows to +inf, as libm's
                want = gf / (1.0 + ex_) * uf
                got = res["act"][r, j, n]
                assert abs(got - want) <= 1e-12 * max(1.0, abs(want)), (r, j, n, got, want)


def test_generator_draws_finite_codes_and_the_scale_range():
    codes, scales = synth.coded_activations(5, 1, 8, 256, -6, -2)
    assert codes.shape == (8, 256) and scales.shape == (8, 8)
    assert not np.any(np.isin(codes, [0x7F, 0xFF]))
    assert scales.min() >= 121 and scales.max() <= 125
    assert len(np.unique(codes)) > 200
