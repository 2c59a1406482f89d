"""Pins of the oracle's bf16 storage step (or_round_bf16) and of the layer with act stored as bf16.

- torch's float32 -> bfloat16 conversion (round to nearest even) on float32-exact values:
  ties at several exponents, the values around them, subnormals, the overflow edge;
- hand-worked cases where rounding float64 through float32 first would give another
  answer (the oracle rounds once, from the exact value);
- exact rational rounding of random float64 values (Fraction arithmetic);
- the layer with act_bf16: its act is the plain layer's act rounded, and its out is the
  float64 down projection of that rounded act.
"""
import math
from fractions import Fraction

import numpy as np
import torch

import oracle
import synth


def _torch_round(vals_f32):
    t = torch.tensor(np.asarray(vals_f32, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def test_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(41)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    # ties and neighbours: low 16 bits 0x8000 (tie), 0x7FFF, 0x8001, with even and odd bf16 lsb
    base = rng.integers(0, 2 ** 16, size=2000, dtype=np.uint64).astype(np.uint32) << np.uint32(16)
    extra = np.concatenate([(base | np.uint32(lo)).view(np.float32) for lo in (0x8000, 0x7FFF, 0x8001, 0x0000)])
    extra = extra[np.isfinite(extra)]
    vals = np.concatenate([f, extra, np.array([1e-40, -3e-39, 3.3e38, 3.39e38, -3.39e38], dtype=np.float32)])
    want = _torch_round(vals)
    got = oracle.round_bf16(vals.astype(np.float64))
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all(), vals[~same][:5]
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_round_once_from_the_exact_value():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 (goes to even: 1); anything above it
    # goes up, even if rounding to float32 first would land on the tie.
    assert oracle.round_bf16(1 + 2 ** -8) == 1.0
    assert oracle.round_bf16(1 + 2 ** -8 + 2 ** -40) == 1 + 2 ** -7
    assert oracle.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6          # tie, odd lsb -> up
    assert oracle.round_bf16(-(1 + 2 ** -8 - 2 ** -40)) == -1.0
    assert oracle.round_bf16(2.0 ** 128 * (1 - 2 ** -9)) == math.inf   # halfway past the largest bf16
    assert oracle.round_bf16(2.0 ** 128 * (1 - 2 ** -9) - 2.0 ** 100) == 2.0 ** 127 * (2 - 2 ** -7)
    assert oracle.round_bf16(2.0 ** -134) == 0.0                       # half the smallest subnormal, even
    assert oracle.round_bf16(2.0 ** -134 * 1.5) == 2.0 ** -133
    assert math.copysign(1.0, oracle.round_bf16(-0.0)) == -1.0
    assert math.isnan(oracle.round_bf16(math.nan))


def _exact_round(v: float) -> Fraction:
    """Nearest multiple of the bf16 step of |v| (8 significant bits), ties to even."""
    a = Fraction(abs(v))
    e = math.frexp(abs(v))[1]
    q = max(e - 8, -133)
    step = Fraction(2) ** q
    n, rem = divmod(a, step)
    if rem > step / 2 or (rem == step / 2 and n % 2 == 1):
        n += 1
    r = n * step
    return -r if v < 0 else r


def test_round_matches_exact_rationals():
    rng = np.random.default_rng(42)
    vals = rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, size=3000)
    got = oracle.round_bf16(vals)
    for v, g in zip(vals, got):
        assert Fraction(g) == _exact_round(float(v)), v


def test_layer_with_bf16_act():
    cfg = synth.CONFIGS["tiny"]
    x, lg = synth.layer_inputs(cfg, 0, plant=False)
    ex = {e: synth.layer_expert(cfg, 0, e) for e in range(cfg.E)}
    plain = oracle.layer(x, lg, ex, cfg.H, cfg.I, cfg.E, cfg.k)
    b16 = oracle.layer(x, lg, ex, cfg.H, cfg.I, cfg.E, cfg.k, act_bf16=True)
    assert np.array_equal(b16["act"], oracle.round_bf16(plain["act"]))
    assert np.array_equal(b16["topk_id"], plain["topk_id"])
    for r in range(cfg.R):
        for j in range(cfg.k):
            e = int(b16["topk_id"][r, j])
            d = oracle.matvec(ex[e]["down_codes"], ex[e]["down_scales"], b16["act"][r, j])
            assert np.array_equal(b16["out"][r, j], d)
        assert np.array_equal(b16["y"][r], oracle.combine(b16["topk_w"][r], b16["out"][r]))
    # rounding act moves out by about 2^-9 relative, not more
    rel = np.abs(b16["out"] - plain["out"]).max() / np.abs(plain["out"]).max()
    assert 0 < rel < 2e-3
