"""GPU: the dense FP8 projection (xp_fp8_pack, xp_fp8_rows) against the oracle, and its
invariance contract.

Values: per-row tolerance against the float64 oracle (max |gpu - ref| / max |ref| over each
row's outputs <= 5e-5; derivation at TOL). The products are exact (E4M3FN values are bf16 values), so
one-hot rows must read back weight x scale exactly. Invariance, bit for bit: a row's
outputs do not depend on how many rows share the launch (every count 1..17 and 33),
on the launch form (waves per 16 columns), or on NaN/Inf planted in other rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from fp4_routed_expert_xp_amd import xp

from gpu_helpers import log, rel_err_rows, to_dev

pytestmark = pytest.mark.gpu

# Each output is exact products summed by four fp32 matrix-core steps (a few roundings
# each), one scale multiply and at most log2(64) = 6 tree adds: under 16 roundings of
# at most 2^-24 relative to sum |x w s|, and for these N(0,1) rows sum |x w s| stays
# within about sqrt(K)/3 <= 30 times max |y| of the row (K <= 8192): 16 * 6e-8 * 30
# is about 3e-5. Measured: about 2e-7.
TOL = 5e-5
SEED = 3001


class Fp8Matrix:
    """One seeded FP8 projection on the GPU: plain bytes, packed bytes and scales."""

    def __init__(self, N, K, layer=0):
        self.N, self.K = N, K
        self.w = synth.fp8_weights(SEED, layer, N, K)
        self.s = synth.fp8_scales(SEED, layer, N, K)
        self.set(self.w)

    def set(self, w):
        self.w = w
        self.w_dev = torch.from_numpy(w).cuda()
        self.packed = torch.empty(xp.xp_fp8_packed_bytes(self.N, self.K), dtype=torch.uint8, device="cuda")
        xp.xp_fp8_pack(self.w_dev, self.packed)
        self.s_dev = torch.from_numpy(self.s).cuda()

    def run(self, x_bits, slices=0):
        R = x_bits.shape[0]
        y = torch.full((max(R, 1), self.N), float("nan"), dtype=torch.float32, device="cuda")
        xp.xp_fp8_rows(R, self.N, self.K, to_dev(x_bits) if R else None, self.packed, self.s_dev, y, slices)
        torch.cuda.synchronize()
        return y.cpu().numpy()[:R]

    def oracle(self, x_bits):
        return oracle.fp8_proj(x_bits, self.w, self.s)

    def run_f32(self, x, slices=0):
        R = x.shape[0]
        y = torch.full((max(R, 1), self.N), float("nan"), dtype=torch.float32, device="cuda")
        xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda() if R else None
        xp.xp_fp8_rows_f32(R, self.N, self.K, xd, self.packed, self.s_dev, y, slices)
        torch.cuda.synchronize()
        return y.cpu().numpy()[:R]


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


SHAPES = [(16, 128), (48, 384), (304, 1536), (576, 4096), (1024, 2048)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_fp8_rows_match_oracle(N, K):
    m = Fp8Matrix(N, K)
    worst = 0.0
    for R in (1, 5, 6, 16, 17, 33):
        log("fp8 N=%d K=%d R=%d" % (N, K, R))
        x = synth.activations(SEED + R, 0, R, K)
        got = m.run(x)
        assert np.all(np.isfinite(got))
        err = rel_err_rows(got, m.oracle(x))
        assert np.all(err <= TOL), (R, float(err.max()))
        worst = max(worst, float(err.max()))
    log("  worst per-row relative error %.2e" % worst)


def test_fp8_largest_k_and_many_row_tiles():
    """K = 8192 (64 blocks: 16 slices of four) and up to 100 rows (seven 16-row tiles,
    the weights held in registers across them)."""
    m = Fp8Matrix(64, 8192, layer=3)
    for R in (1, 16, 100):
        x = synth.activations(SEED + 7, R, R, 8192)
        err = rel_err_rows(m.run(x), m.oracle(x))
        assert np.all(err <= TOL), (R, float(err.max()))
    x = synth.activations(SEED + 7, 100, 100, 8192)
    full = m.run(x)
    for r in (0, 47, 99):
        assert np.array_equal(bits(full[r:r + 1]), bits(m.run(x[r:r + 1]))), r


def test_fp8_pack_layout():
    N, K = 48, 384
    m = Fp8Matrix(N, K)
    got = m.packed.cpu().numpy()
    # [tile][block][lane = (q, c)][group][8]: column 16 tile + c, k = 128 block + 32 group + 8 q
    w = m.w.reshape(N // 16, 16, K // 128, 4, 4, 8)           # tile, c, block, group, q, 8
    want = w.transpose(0, 2, 4, 1, 3, 5).reshape(-1)          # tile, block, q, c, group, 8
    assert np.array_equal(got, want)


def test_fp8_one_hot_rows_are_exact():
    # Every non-NaN byte appears; rows are one-hot (bf16 1.0) at k's in different
    # blocks, so each output is one weight times its block scale, exactly.
    N, K = 304, 512
    m = Fp8Matrix(N, K)
    ks = [0, 1, 31, 32, 127, 128, 300, 511, 64, 200, 255, 256, 384, 450, 7, 100, 222]
    x = np.zeros((len(ks), K), dtype=np.uint16)
    for r, k in enumerate(ks):
        x[r, k] = 0x3F80
    got = m.run(x)
    want = m.oracle(x).astype(np.float32)
    assert np.array_equal(bits(got), bits(want))


def test_fp8_nan_weight_poisons_its_column():
    N, K = 48, 256
    m = Fp8Matrix(N, K)
    w = m.w.copy()
    w[5, 17] = 0x7F
    w[40, 200] = 0xFF
    m.set(w)
    x = synth.activations(SEED, 7, 3, K)
    got = m.run(x)
    assert np.all(np.isnan(got[:, [5, 40]]))
    keep = [n for n in range(N) if n not in (5, 40)]
    assert np.all(np.isfinite(got[:, keep]))


@pytest.fixture(scope="module")
def wide():
    return Fp8Matrix(576, 4096, layer=1)


def test_fp8_rows_equal_their_one_row_launch(wide):
    """Every row count 1..17 and 33 (three 16-row tiles): each row's bits equal
    that row launched alone."""
    K = wide.K
    x = synth.activations(SEED, 11, 33, K)
    alone = np.stack([wide.run(x[r:r + 1])[0] for r in range(33)])
    for R in list(range(1, 18)) + [33]:
        got = wide.run(x[:R])
        assert np.array_equal(bits(got), bits(alone[:R])), R
    # a row's bits do not depend on its position in the launch either
    p = np.random.default_rng(3).permutation(33)
    assert np.array_equal(bits(wide.run(x[p])), bits(alone[p]))


def test_fp8_forms_are_bit_equal():
    """Waves per 16 columns (how K is split) do not change a bit: K = 512 (4
    blocks) under 1, 2, 4 slices; K = 1536 (12 blocks, padded to 16) under
    4, 8, 16; K = 4096 under 8, 16."""
    for (N, K), forms in (((64, 512), (1, 2, 4)), ((304, 1536), (4, 8, 16)), ((576, 4096), (8, 16))):
        m = Fp8Matrix(N, K, layer=2)
        for R in (1, 6, 16):
            x = synth.activations(SEED + 50, R, R, K)
            ref = m.run(x, slices=forms[0])
            for f in forms[1:]:
                assert np.array_equal(bits(m.run(x, slices=f)), bits(ref)), (N, K, R, f)
            assert np.array_equal(bits(m.run(x, slices=0)), bits(ref)), (N, K, R, "auto")


def test_fp8_nan_and_inf_stay_in_their_rows(wide):
    """A batch of 16 with NaN planted in row 3 and +Inf in row 7: every other row
    equals its one-row launch; row 3 is NaN everywhere; row 7's non-finite
    pattern is the float64 oracle's."""
    K = wide.K
    x = synth.activations(SEED, 12, 16, K)
    x[3, 1000] = 0x7FC1
    x[7, 2049] = 0x7F80
    got = wide.run(x)
    for r in range(16):
        if r in (3, 7):
            continue
        assert np.array_equal(bits(got[r]), bits(wide.run(x[r:r + 1])[0])), r
    assert np.all(np.isnan(got[3]))
    ref = wide.oracle(x[7:8])[0]
    assert np.array_equal(np.isnan(got[7]), np.isnan(ref))
    assert np.array_equal(np.isposinf(got[7]), np.isposinf(ref))
    assert np.array_equal(np.isneginf(got[7]), np.isneginf(ref))


def test_fp8_empty_and_errors():
    m = Fp8Matrix(16, 128)
    assert m.run(np.zeros((0, 128), dtype=np.uint16)).shape == (0, 16)
    x = to_dev(np.zeros((1, 128), dtype=np.uint16))
    y = torch.zeros((1, 16), dtype=torch.float32, device="cuda")
    with pytest.raises(xp.XPError) as ei:
        xp.xp_fp8_rows(1, 16, 128, x, m.packed, m.s_dev, y, slices=2)   # P = 1: at most one slice
    assert ei.value.status == xp.XP_ERR_SHAPE


def f32_rows(seed, R, K):
    return (np.random.default_rng(seed).standard_normal((R, K)) * 2).astype(np.float32)


@pytest.mark.parametrize("N,K", [(48, 384), (576, 4096), (64, 8192)])
def test_fp8_f32_rows_match_oracle(N, K):
    m = Fp8Matrix(N, K, layer=4)
    for R in (1, 6, 16, 33):
        x = f32_rows(SEED + R, R, K)
        err = rel_err_rows(m.run_f32(x), oracle.fp8_proj_f32(x, m.w, m.s))
        assert np.all(err <= TOL), (R, float(err.max()))


def test_fp8_f32_rows_invariance():
    """Row counts 1..17, every form, and planted NaN / +Inf rows: each row's bits
    equal its one-row launch."""
    m = Fp8Matrix(304, 1536, layer=5)
    x = f32_rows(SEED, 17, 1536)
    x[4, 100] = np.nan
    x[9, 1000] = np.inf
    alone = np.stack([m.run_f32(x[r:r + 1])[0] for r in range(17)])
    for R in range(1, 18):
        assert np.array_equal(bits(m.run_f32(x[:R])), bits(alone[:R])), R
    for f in (4, 8, 16):
        assert np.array_equal(bits(m.run_f32(x, slices=f)), bits(alone)), f
    assert np.all(np.isnan(alone[4]))
    ref = oracle.fp8_proj_f32(x[9:10], m.w, m.s)[0]
    assert np.array_equal(np.isnan(alone[9]), np.isnan(ref))
    assert np.array_equal(np.isposinf(alone[9]), np.isposinf(ref))


def test_fp8_f32_one_hot_rows_are_exact():
    """One-hot fp32 rows (parts 1, 0, 0) read back weight x block scale exactly."""
    m = Fp8Matrix(304, 512, layer=6)
    ks = [0, 5, 127, 128, 300, 511]
    x = np.zeros((len(ks), 512), dtype=np.float32)
    for r, k in enumerate(ks):
        x[r, k] = 1.0
    assert np.array_equal(bits(m.run_f32(x)), bits(oracle.fp8_proj_f32(x, m.w, m.s).astype(np.float32)))


@pytest.mark.parametrize("K,Ns", [(4096, (576, 1536, 4096)), (512, (16, 48, 304, 1024, 16, 32, 64, 128)),
                                  (2048, (1024,))])
def test_fp8_rows_multi_equals_separate_launches(K, Ns):
    """One launch over several matrices that share x: each matrix's y bit-equal to
    its own xp_fp8_rows launch, at row counts 1, 5, 16 and 33, with NaN and +Inf
    planted in other rows, in the default form and in the form with the fewest
    waves per workgroup (four blocks per wave)."""
    mats = [Fp8Matrix(N, K, layer=i) for i, N in enumerate(Ns)]
    P = 1
    while P < K // 128:
        P *= 2
    for R in (1, 5, 16, 33):
        x = synth.activations(SEED + 70 + R, 0, R, K)
        if R >= 2:
            x, _, _ = synth.plant_nan_inf(SEED + 70, R, x)
        for slices in (0, max(1, P // 4)):
            ys = [torch.full((R, m.N), float("nan"), dtype=torch.float32, device="cuda") for m in mats]
            xp.xp_fp8_rows_multi(R, K, to_dev(x), [(m.packed, m.s_dev, y) for m, y in zip(mats, ys)], slices)
            torch.cuda.synchronize()
            for m, y in zip(mats, ys):
                assert np.array_equal(bits(y.cpu().numpy()), bits(m.run(x, slices))), (K, m.N, R, slices)


def test_fp8_rows_multi_refusals():
    m = Fp8Matrix(16, 128)
    x = to_dev(synth.activations(SEED, 0, 1, 128))
    y = torch.empty((1, 16), dtype=torch.float32, device="cuda")
    with pytest.raises(xp.XPError) as ei:
        xp.xp_fp8_rows_multi(1, 128, x, [(m.packed, m.s_dev, y)] * 9)
    assert ei.value.status == xp.XP_ERR_SHAPE
    with pytest.raises(xp.XPError) as ei:
        xp.xp_fp8_rows_multi(1, 128, x, [])
    assert ei.value.status == xp.XP_ERR_SHAPE
    xp.xp_fp8_rows_multi(0, 128, None, [(m.packed, m.s_dev, y)])   # no rows: nothing to do
