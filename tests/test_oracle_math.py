"""Pins of the oracle's float64 layer math and of its fp32 chain replay.

Each test checks the oracle against something other than itself: exact
rational brute force, closed forms, invariants, hand-built cases whose result
follows from the rounding rules, or numpy's own float64 matmul on a matrix
decoded through torch's float8 codec.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import brute

E2M1_TABLE = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def _rand_matrix(rng, N, K, emin=-3, emax=2):
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    e = rng.integers(emin, emax + 1, size=(N, K // 32))
    scales = ((e + 7) << 3).astype(np.uint8)
    return codes, scales


def _independent_decode(codes, scales):
    """Decode with torch's float8_e4m3fn and the OCP E2M1 table (no oracle code)."""
    lo = E2M1_TABLE[codes & 15]
    hi = E2M1_TABLE[codes >> 4]
    w = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)
    s = torch.from_numpy(scales.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return w * np.repeat(s, 32, axis=1)


def test_matvec_brute_force_exact():
    rng = np.random.default_rng(1)
    N, K = 3, 64
    codes, scales = _rand_matrix(rng, N, K)
    x_bits = synth.activations(9, 0, 1, K)[0]
    xq = [brute.bf16(int(b)) for b in x_bits]
    exact = brute.matvec(codes, scales, xq)
    bound = brute.abs_matvec(codes, scales, xq)
    y = oracle.matvec(codes, scales, oracle.bf16_to_f64(x_bits))
    for n in range(N):
        err = abs(Fraction(y[n]) - exact[n])
        assert err <= bound[n] * Fraction(K + 1, 2 ** 53), (n, float(err))


def test_matvec_one_hot_reads_each_weight():
    rng = np.random.default_rng(2)
    N, K = 4, 96
    codes, scales = _rand_matrix(rng, N, K)
    for k in range(K):
        x = np.zeros(K)
        x[k] = 1.0
        y = oracle.matvec(codes, scales, x)
        for n in range(N):
            assert y[n] == float(brute.weight(codes, scales, n, k)), (n, k)


def test_matvec_layout_hand_example():
    # one row, K = 32: byte 0 = 0x21 -> k0 = code 1 (0.5), k1 = code 2 (1.0); byte 1 = 0xF7 -> k2 = 6, k3 = -6
    codes = np.zeros((1, 16), dtype=np.uint8)
    codes[0, 0] = 0x21
    codes[0, 1] = 0xF7
    scales = np.array([[0x40]], dtype=np.uint8)   # 2.0
    x = np.zeros(32)
    x[:4] = [1.0, 10.0, 100.0, 1000.0]
    y = oracle.matvec(codes, scales, x)
    assert y[0] == 2.0 * (0.5 * 1 + 1.0 * 10 + 6.0 * 100 - 6.0 * 1000)


def test_matvec_constant_codes_unit_scales():
    K = 256
    for c in range(16):
        codes = np.full((2, K // 2), c | (c << 4), dtype=np.uint8)
        scales = np.full((2, K // 32), 0x38, dtype=np.uint8)
        x = synth.bf16_bits_to_f32(synth.activations(4, c, 1, K)[0]).astype(np.float64)
        y = oracle.matvec(codes, scales, x)
        want = E2M1_TABLE[c] * x.sum()
        assert np.allclose(y, want, rtol=1e-12, atol=1e-12)


def test_matvec_matches_numpy_on_independent_decode():
    rng = np.random.default_rng(3)
    N, K = 64, 512
    codes, scales = _rand_matrix(rng, N, K, -6, 0)
    x = rng.standard_normal(K)
    y = oracle.matvec(codes, scales, x)
    ref = _independent_decode(codes, scales) @ x
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_matvec_scale_doubling_doubles_group():
    rng = np.random.default_rng(4)
    N, K = 5, 128
    codes, scales = _rand_matrix(rng, N, K, -3, 1)
    x = rng.standard_normal(K)
    base = oracle.matvec(codes, scales, x)
    s2 = scales.copy()
    s2[:, 2] += 8                      # exponent + 1 -> scale x 2 on group 2
    x_g = np.zeros(K)
    x_g[64:96] = x[64:96]
    part = oracle.matvec(codes, scales, x_g)
    y2 = oracle.matvec(codes, s2, x)
    assert np.allclose(y2, base + part, rtol=1e-12, atol=1e-12)


def test_swiglu_values():
    g = np.array([0.0, 1.0, -1.0, 30.0, -30.0, 2.5])
    u = np.array([3.0, 1.0, 1.0, 2.0, 2.0, -4.0])
    a = oracle.swiglu(g, u)
    sig = [0.5, 0.7310585786300049, 0.2689414213699951]
    assert a[0] == 0.0
    assert abs(a[1] - sig[1]) < 1e-15
    assert abs(a[2] + sig[2]) < 1e-15
    assert abs(a[3] - 60.0) < 1e-11
    assert abs(a[4]) < 1e-11
    assert abs(a[5] - (-4.0 * 2.5 / (1 + math.exp(-2.5)))) < 1e-14


def test_combine_closed_form():
    out = np.arange(12, dtype=np.float64).reshape(3, 4)
    w = np.array([0.5, 0.25, 0.25])
    y = oracle.combine(w, out)
    assert list(y) == [0.5 * 0 + 0.25 * 4 + 0.25 * 8, 0.5 + 0.25 * 5 + 0.25 * 9,
                       0.5 * 2 + 0.25 * 6 + 0.25 * 10, 0.5 * 3 + 0.25 * 7 + 0.25 * 11]


# -------------------------------------------------------------- fp32 replay
def test_chain32_equals_float64_on_exact_inputs():
    rng = np.random.default_rng(5)
    N, K = 32, 4096
    codes, scales = _rand_matrix(rng, N, K, -6, 0)
    x = rng.integers(-4, 5, size=K).astype(np.float32)      # integers: every fp32 sum exact
    y32 = oracle.chain32(codes, scales, x)
    y64 = oracle.matvec(codes, scales, x.astype(np.float64))
    assert np.array_equal(y32.astype(np.float64), y64)


def test_chain32_within_rounding_bound():
    rng = np.random.default_rng(6)
    N, K = 16, 1024
    codes, scales = _rand_matrix(rng, N, K, -6, 0)
    x = synth.bf16_bits_to_f32(synth.activations(8, 0, 1, K)[0])
    y32 = oracle.chain32(codes, scales, x).astype(np.float64)
    y64 = oracle.matvec(codes, scales, x.astype(np.float64))
    mag = np.abs(_independent_decode(codes, scales)) @ np.abs(x.astype(np.float64))
    depth = 32 + K // 32 // 8 + 3
    u = 2.0 ** -24
    assert np.all(np.abs(y32 - y64) <= depth * u / (1 - depth * u) * mag)


def _one_hot_groups(group_values, K):
    """x with x[32g] = value_g and w = 1.0 at those k, so each group's chain is exactly value_g."""
    N = 1
    codes = np.zeros((N, K // 2), dtype=np.uint8)
    scales = np.full((N, K // 32), 0x38, dtype=np.uint8)
    x = np.zeros(K, dtype=np.float32)
    for g, v in enumerate(group_values):
        codes[0, 16 * g] = 0x02          # k = 32g -> code 2 = 1.0
        x[32 * g] = v
    return codes, scales, x


def test_chain32_tree_shape():
    # partials p0..p7 = 2^24, 1, 1, -2^24, 0...: the pairwise tree gives
    # (2^24 + 1) + (1 - 2^24) = 2^24 + (-2^24 + 1) = 1, a left-to-right sum gives 0.
    K = 32 * 8
    codes, scales, x = _one_hot_groups([2.0 ** 24, 1.0, 1.0, -(2.0 ** 24), 0, 0, 0, 0], K)
    assert oracle.chain32(codes, scales, x)[0] == 1.0
    # the other half of the tree: p4..p7
    codes, scales, x = _one_hot_groups([0, 0, 0, 0, 2.0 ** 24, 1.0, 1.0, -(2.0 ** 24)], K)
    assert oracle.chain32(codes, scales, x)[0] == 1.0


def test_chain32_group_to_partial_mapping():
    # groups 0 and 8 both feed partial 0 (in that order); group 1 feeds partial 1.
    # partial0 = (2^24 + 1) -> 2^24 (ties to even), partial1 = -2^24 -> total 0.
    # Were group 8 sent to partial 1, the total would be (2^24) + (1 - 2^24) = 1.
    K = 32 * 16
    vals = [0.0] * 16
    vals[0], vals[8], vals[1] = 2.0 ** 24, 1.0, -(2.0 ** 24)
    codes, scales, x = _one_hot_groups(vals, K)
    assert oracle.chain32(codes, scales, x)[0] == 0.0


def test_chain32_scale_is_fused_after_the_chain():
    # group 0 chain = 1 + 2^-23, scale 1.125 (0x39); group 8 (same partial) adds
    # an accumulator value so that fused and unfused rounding differ.
    K = 32 * 16
    codes = np.zeros((1, K // 2), dtype=np.uint8)
    scales = np.full((1, K // 32), 0x38, dtype=np.uint8)
    x = np.zeros(K, dtype=np.float32)
    codes[0, 0] = 0x02
    x[0] = -1.0                                   # group 0: p = -1, scale 1 -> partial0 = -1
    codes[0, 16 * 8] = 0x02
    x[32 * 8] = np.float32(1.0 + 2.0 ** -23)      # group 8: p = 1 + 2^-23
    scales[0, 8] = 0x39                           # 1.125
    exact = Fraction(1) + Fraction(1, 2 ** 23)
    fused = float(np.float32(float(exact * Fraction(9, 8) - 1)))
    unfused = float(np.float32(np.float32(np.float32(exact) * np.float32(1.125)) - np.float32(1.0)))
    assert fused != unfused
    assert oracle.chain32(codes, scales, x)[0] == fused


def test_chain32_partials_start_from_plus_zero():
    # a group whose products are all -0 must leave its partial at +0, so the
    # output is +0, not -0 (a partial started from -0 would give -0).
    K = 32
    codes = np.full((1, 16), 0x88, dtype=np.uint8)   # every weight -0
    scales = np.full((1, 1), 0x38, dtype=np.uint8)
    x = np.ones(K, dtype=np.float32)
    y = oracle.chain32(codes, scales, x)[0]
    assert y == 0.0 and math.copysign(1.0, y) == 1.0


def test_chain32_groups_enter_a_partial_in_ascending_order():
    # partial 0 takes groups 0, 8, 16 = 1, 2^24, -2^24: ascending gives
    # (1 + 2^24) - 2^24 = 0, descending would give (-2^24 + 2^24) + 1 = 1.
    K = 32 * 24
    vals = [0.0] * 24
    vals[0], vals[8], vals[16] = 1.0, 2.0 ** 24, -(2.0 ** 24)
    codes, scales, x = _one_hot_groups(vals, K)
    assert oracle.chain32(codes, scales, x)[0] == 0.0


def test_combine32_is_fused_chain_in_slot_order():
    # slot 0: 1 * -1 -> y = -1; slot 1: (1 + 2^-23)(1 + 2^-22) fused into -1
    # gives 3*2^-23 + 2^-45 exactly; an unfused product, or the slots taken in
    # the other order, gives 3*2^-23.
    w = np.array([1.0, 1.0 + 2 ** -23], dtype=np.float32)
    out = np.array([[-1.0], [1.0 + 2 ** -22]], dtype=np.float32)
    y = oracle.combine32(w, out)[0]
    assert y == 3 * 2.0 ** -23 + 2.0 ** -45
