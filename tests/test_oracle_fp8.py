"""Pins of the oracle's dense FP8 projection (or_fp8_proj) against things other than itself.

- exact rational brute force on a tiny case (brute.e4m3 / brute.bf16, written apart
  from oracle.c), within the float64 summation bound;
- one-hot rows, which must read back each weight times its own 128 x 128 block's
  scale exactly (a transposed operand or a swapped block index fails here);
- a hand-worked example;
- numpy's float64 matmul on a matrix decoded through torch's float8_e4m3fn codec.
"""
from fractions import Fraction

import numpy as np
import torch

import oracle
import synth
from oracle import brute

BF16_ONE = 0x3F80


def _torch_decode(w):
    return torch.from_numpy(np.ascontiguousarray(w)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _block_scales(s, N, K):
    """[ceil(N/128)][K/128] -> [N][K] by repeating each block's scale."""
    full = np.repeat(np.repeat(s.astype(np.float64), 128, axis=0), 128, axis=1)
    return full[:N, :K]


def _valid_bytes(rng, shape):
    b = rng.integers(0, 254, size=shape)
    return np.where(b >= 0x7F, b + 1, b).astype(np.uint8)   # skip 0x7F; 0xFF is out of range


def test_fp8_brute_force_exact():
    rng = np.random.default_rng(11)
    R, N, K = 2, 3, 256
    w = _valid_bytes(rng, (N, K))
    s = np.array([[2.0 ** -3, 2.0 ** 2]], dtype=np.float32)
    x = synth.activations(21, 0, R, K)
    y = oracle.fp8_proj(x, w, s)
    for r in range(R):
        xq = [brute.bf16(int(b)) for b in x[r]]
        for n in range(N):
            terms = [xq[k] * brute.e4m3(int(w[n, k])) * Fraction(float(s[0, k // 128])) for k in range(K)]
            exact = sum(terms, Fraction(0))
            bound = sum((abs(t) for t in terms), Fraction(0)) * Fraction(K + 1, 2 ** 53)
            assert abs(Fraction(y[r, n]) - exact) <= bound, (r, n)


def test_fp8_one_hot_reads_each_weight_and_its_block_scale():
    # N = 300 leaves a ragged third block of output columns; K = 384 has three
    # blocks along k; every scale is a different power of two.
    rng = np.random.default_rng(12)
    N, K = 300, 384
    w = _valid_bytes(rng, (N, K))   # every non-NaN byte
    s = np.array([[2.0 ** e for e in row] for row in ([-4, 0, 3], [1, -2, 5], [-1, 2, -6])], dtype=np.float32)
    ks = [0, 1, 127, 128, 200, 255, 256, 383]
    x = np.zeros((len(ks), K), dtype=np.uint16)
    for r, k in enumerate(ks):
        x[r, k] = BF16_ONE
    y = oracle.fp8_proj(x, w, s)
    ref = _torch_decode(w)
    for r, k in enumerate(ks):
        for n in range(N):
            assert y[r, n] == ref[n, k] * float(s[n // 128, k // 128]), (r, n, k)


def test_fp8_nan_weight_poisons_its_column_only():
    # 0 * NaN is NaN, so a NaN byte (0x7F or 0xFF) makes its output column NaN
    # for every row, even where x is zero; the other columns are unchanged.
    rng = np.random.default_rng(15)
    R, N, K = 3, 40, 128
    w = _valid_bytes(rng, (N, K))
    s = np.array([[1.0]], dtype=np.float32)
    x = synth.activations(24, 0, R, K)
    clean = oracle.fp8_proj(x, w, s)
    w[7, 5] = 0x7F
    w[30, 100] = 0xFF
    y = oracle.fp8_proj(x, w, s)
    assert np.all(np.isnan(y[:, [7, 30]]))
    keep = [n for n in range(N) if n not in (7, 30)]
    assert np.array_equal(y[:, keep], clean[:, keep])


def test_fp8_hand_example():
    # K = 256 (two blocks). Row 0 of W is 1.0 (0x38) everywhere; row 1 is +2.0
    # (0x40) on even k and -2.0 (0xC0) on odd k. x = 1.5 (0x3FC0) on the first
    # block and 0.5 (0x3F00) on the second. Scales: 0.25 for block 0, 4.0 for block 1.
    #   y[0] = 128 * 1.5 * 1 * 0.25 + 128 * 0.5 * 1 * 4 = 48 + 256 = 304
    #   y[1] = 0 (pairs +2, -2 cancel in each block)
    # Row 2 of W puts 448 (0x7E) at k = 3 and zero (0x00) elsewhere:
    #   y[2] = 1.5 * 448 * 0.25 = 168
    K = 256
    w = np.zeros((3, K), dtype=np.uint8)
    w[0, :] = 0x38
    w[1, 0::2] = 0x40
    w[1, 1::2] = 0xC0
    w[2, 3] = 0x7E
    x = np.zeros((1, K), dtype=np.uint16)
    x[0, :128] = 0x3FC0
    x[0, 128:] = 0x3F00
    s = np.array([[0.25, 4.0]], dtype=np.float32)
    y = oracle.fp8_proj(x, w, s)
    assert y.tolist() == [[304.0, 0.0, 168.0]]


def test_fp8_matches_numpy_on_independent_decode():
    rng = np.random.default_rng(13)
    R, N, K = 3, 200, 384
    w = _valid_bytes(rng, (N, K))
    s = (2.0 ** rng.integers(-8, 3, size=(2, 3))).astype(np.float32)
    x = synth.activations(22, 0, R, K)
    W = _torch_decode(w) * _block_scales(s, N, K)
    ref = synth.bf16_bits_to_f32(x).astype(np.float64) @ W.T
    y = oracle.fp8_proj(x, w, s)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_fp8_rows_are_independent():
    # Each output row depends on its own row of x only: permuting rows permutes y.
    rng = np.random.default_rng(14)
    R, N, K = 5, 16, 128
    w = _valid_bytes(rng, (N, K))
    s = np.array([[0.5]], dtype=np.float32)
    x = synth.activations(23, 0, R, K)
    p = rng.permutation(R)
    assert np.array_equal(oracle.fp8_proj(x[p], w, s), oracle.fp8_proj(x, w, s)[p])


def test_fp8_f32_rows_match_numpy_and_the_bf16_form():
    rng = np.random.default_rng(16)
    R, N, K = 3, 144, 256
    w = _valid_bytes(rng, (N, K))
    s = (2.0 ** rng.integers(-6, 2, size=(2, 2))).astype(np.float32)
    x = (rng.standard_normal((R, K)) * 3).astype(np.float32)
    W = _torch_decode(w) * _block_scales(s, N, K)
    ref = x.astype(np.float64) @ W.T
    y = oracle.fp8_proj_f32(x, w, s)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # rows whose values are bf16 values give the bf16 form's result exactly
    xb = synth.activations(25, 0, R, K)
    assert np.array_equal(oracle.fp8_proj_f32(synth.bf16_bits_to_f32(xb), w, s), oracle.fp8_proj(xb, w, s))
