"""GPU: values against the oracle.

- The chains, scaled fmas and the eight-leaf tree are bit-exact against the
  oracle's fp32 replay (gate/up before the epilogue, down on a given act,
  combine on given outputs).
- act, out and y are within the stated tolerance of the float64 oracle:
  per row, max|gpu - ref| / max|ref| <= 1e-3 over the oracle's finite entries,
  with non-finite entries of the same class.
- On exact inputs (integer activations, power-of-two scales) every fp32 sum
  is exact, so the projections equal float64 bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from fp4_routed_expert_xp_amd import xp

from gpu_helpers import DeviceLayer, bits, log, read_plan, rel_err_rows, run_fused, run_path, same_class, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3
TINY = synth.CONFIGS["tiny"]


@pytest.fixture(scope="module")
def tiny_layer():
    return DeviceLayer(TINY, 0)


@pytest.fixture(scope="module")
def release_layer():
    cfg = synth.CONFIGS["one_row"]
    log("materialising release-width layer 0 (256 experts)")
    return DeviceLayer(cfg, 0)


def _oracle_layer(layer: DeviceLayer, x, lg):
    ids, _ = oracle.route(lg, layer.cfg.k)
    ex = {int(e): layer.host_expert(int(e)) for e in np.unique(ids)}
    return oracle.layer(x, lg, ex, layer.cfg.H, layer.cfg.I, layer.cfg.E, layer.cfg.k)


def _check_values(res, ref, R):
    assert np.array_equal(res["topk_id"], ref["topk_id"])
    for name in ("act", "out", "y"):
        err = rel_err_rows(res[name], ref[name])
        assert np.all(err <= TOL), (name, err)
        assert same_class(res[name], ref[name]), name


def _check_chains(layer: DeviceLayer, x, res, rows):
    """g, u bit-equal to the fp32 replay for the given rows."""
    k = layer.cfg.k
    xf = synth.bf16_bits_to_f32(x)
    for r in rows:
        for j in range(k):
            e = layer.host_expert(int(res["topk_id"][r, j]))
            g = oracle.chain32(e["gate_codes"], e["gate_scales"], xf[r])
            u = oracle.chain32(e["up_codes"], e["up_scales"], xf[r])
            assert np.array_equal(bits(res["g"][r, j]), bits(g)), (r, j)
            assert np.array_equal(bits(res["u"][r, j]), bits(u)), (r, j)


# ------------------------------------------------------------------ tiny widths
@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 9, 16, 64, 65, 130])
def test_tiny_layer_matches_oracle(tiny_layer, R):
    log("tiny R=%d" % R)
    x = synth.activations(TINY.seed, R, R, TINY.H)
    lg = synth.logits(TINY.seed, R, R, TINY.E)
    res = run_path(tiny_layer, x, lg, split=True, canary=True)
    ref = _oracle_layer(tiny_layer, x, lg)
    _check_values(res, ref, R)
    _check_chains(tiny_layer, x, res, range(R))


def test_tiny_planted_nan_inf(tiny_layer):
    x, lg = synth.layer_inputs(TINY, 0, plant=True)
    res = run_path(tiny_layer, x, lg, canary=True)
    ref = _oracle_layer(tiny_layer, x, lg)
    _check_values(res, ref, TINY.R)


@pytest.mark.parametrize("tiers", [((4,), (4,)), ((8,), (8,)), ((2, 4, 8), (2, 4, 8)), ((3, 5, 7), (2, 3))])
def test_tiny_tier_sets(tiny_layer, tiers):
    R = 16
    x = synth.activations(TINY.seed, 100, R, TINY.H)
    lg = synth.logits_same(TINY.seed, 100, R, TINY.E)
    base = run_path(tiny_layer, x, lg)
    xp.xp_set_tiers(list(tiers[0]), list(tiers[1]))
    try:
        other = run_path(tiny_layer, x, lg)
    finally:
        xp.xp_set_tiers(None, None)
    for name in ("act", "out", "y"):
        assert np.array_equal(bits(base[name]), bits(other[name])), name


def test_empty_batch(tiny_layer):
    d = tiny_layer.d
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    xp.xp_route_bucket(d, 0, None, None, None, ws)
    xp.xp_gateup_rows(d, 0, None, tiny_layer.table, ws, None)
    xp.xp_down_rows(d, 0, None, tiny_layer.table, ws, None)
    xp.xp_combine(d, 0, None, None, None)
    torch.cuda.synchronize()


def test_outputs_written_exactly_in_bounds(tiny_layer):
    """Canary guards around act/out/y stay untouched; every real (row, slot) is written."""
    d = tiny_layer.d
    R, k, H, I = 5, d.top_k, d.hidden, d.inter
    x = to_dev(synth.activations(3, 3, R, H))
    lg = to_dev(synth.logits_same(3, 3, R, d.n_experts))
    ws = torch.zeros(xp.xp_workspace_bytes(d, R), dtype=torch.uint8, device="cuda")
    ids = torch.empty((R, k), dtype=torch.int32, device="cuda")
    w = torch.empty((R, k), dtype=torch.float32, device="cuda")
    pad = 4096
    canary = -12345.0
    act = torch.full((R * k * I + 2 * pad,), canary, device="cuda")
    out = torch.full((R * k * H + 2 * pad,), canary, device="cuda")
    xp.xp_route_bucket(d, R, lg, ids, w, ws)
    xp.xp_gateup_rows(d, R, x, tiny_layer.table, ws, act[pad:pad + R * k * I])
    xp.xp_down_rows(d, R, act[pad:pad + R * k * I], tiny_layer.table, ws, out[pad:pad + R * k * H])
    torch.cuda.synchronize()
    a, o = act.cpu().numpy(), out.cpu().numpy()
    assert np.all(a[:pad] == canary) and np.all(a[-pad:] == canary)
    assert np.all(o[:pad] == canary) and np.all(o[-pad:] == canary)
    assert not np.any(a[pad:-pad] == canary) and not np.any(o[pad:-pad] == canary)


def test_exact_inputs_are_bit_equal_to_float64(tiny_layer):
    """Integer activations and power-of-two scales: g, u and out equal float64 exactly."""
    d = tiny_layer.d
    R = 4
    rng = np.random.default_rng(11)
    xi = rng.integers(-4, 5, size=(R, d.hidden)).astype(np.float32)
    x = synth.f32_to_bf16_bits(xi)
    lg = synth.logits(11, 0, R, d.n_experts)
    res = run_path(tiny_layer, x, lg, split=True)
    for r in range(R):
        for j in range(d.top_k):
            e = tiny_layer.host_expert(int(res["topk_id"][r, j]))
            g64 = oracle.matvec(e["gate_codes"], e["gate_scales"], xi[r].astype(np.float64))
            u64 = oracle.matvec(e["up_codes"], e["up_scales"], xi[r].astype(np.float64))
            assert np.array_equal(res["g"][r, j].astype(np.float64), g64)
            assert np.array_equal(res["u"][r, j].astype(np.float64), u64)
    # down on an integer act (given, not computed): out equals float64 exactly
    ai = rng.integers(-4, 5, size=(R, d.top_k, d.inter)).astype(np.float32)
    ws = to_dev(res["ws"])
    out = torch.empty((R, d.top_k, d.hidden), dtype=torch.float32, device="cuda")
    xp.xp_down_rows(d, R, to_dev(ai), tiny_layer.table, ws, out)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for r in range(R):
        for j in range(d.top_k):
            e = tiny_layer.host_expert(int(res["topk_id"][r, j]))
            o64 = oracle.matvec(e["down_codes"], e["down_scales"], ai[r, j].astype(np.float64))
            assert np.array_equal(out[r, j].astype(np.float64), o64)


def test_down_and_combine_bit_equal_to_fp32_replay(tiny_layer):
    d = tiny_layer.d
    R = 7
    x = synth.activations(21, 0, R, d.hidden)
    lg = synth.logits(21, 0, R, d.n_experts)
    res = run_path(tiny_layer, x, lg)
    rng = np.random.default_rng(21)
    a = rng.standard_normal((R, d.top_k, d.inter)).astype(np.float32)
    ws = to_dev(res["ws"])
    out = torch.empty((R, d.top_k, d.hidden), dtype=torch.float32, device="cuda")
    xp.xp_down_rows(d, R, to_dev(a), tiny_layer.table, ws, out)
    o = rng.standard_normal((R, d.top_k, d.hidden)).astype(np.float32)
    w = rng.random((R, d.top_k)).astype(np.float32)
    y = torch.empty((R, d.hidden), dtype=torch.float32, device="cuda")
    xp.xp_combine(d, R, to_dev(o), to_dev(w), y)
    torch.cuda.synchronize()
    out, y = out.cpu().numpy(), y.cpu().numpy()
    for r in range(R):
        for j in range(d.top_k):
            e = tiny_layer.host_expert(int(res["topk_id"][r, j]))
            ref = oracle.chain32(e["down_codes"], e["down_scales"], a[r, j])
            assert np.array_equal(bits(out[r, j]), bits(ref)), (r, j)
        assert np.array_equal(bits(y[r]), bits(oracle.combine32(w[r], o[r]))), r


def test_wide_combine_bit_equal_to_fp32_replay():
    # 300 rows of width 4096: 1,228,800 outputs, enough for the four-per-thread
    # form. Every row against the fp32 replay of the slot-order chain, and the
    # bf16 form against that result rounded to nearest even.
    R, H, k = 300, 4096, 8
    d = xp.dims(H, 2048, 256, k)
    rng = np.random.default_rng(33)
    o = rng.standard_normal((R, k, H)).astype(np.float32)
    w = rng.random((R, k)).astype(np.float32)
    y = torch.empty((R, H), dtype=torch.float32, device="cuda")
    y16 = torch.empty((R, H), dtype=torch.int16, device="cuda")
    xp.xp_combine(d, R, to_dev(o), to_dev(w), y)
    xp.xp_combine_y16(d, R, to_dev(o), to_dev(w), y16)
    torch.cuda.synchronize()
    y, y16 = y.cpu().numpy(), y16.cpu().numpy()
    for r in range(R):
        assert np.array_equal(bits(y[r]), bits(oracle.combine32(w[r], o[r]))), r
    assert np.array_equal(y16, synth.f32_to_bf16_bits(y).view(np.int16))


# --------------------------------------------------------------- release widths
@pytest.mark.parametrize("name", ["one_row", "four_same", "sixteen_random"])
def test_release_layer_matches_oracle(release_layer, name):
    """Every row of the workload's seeded input (sixteen random rows with the
    NaN and +Inf planted) against the float64 oracle, on the four-call path and
    on the two-call path (xp_route_gateup, xp_down_combine); the two paths also
    give the same bits."""
    cfg = synth.CONFIGS[name]
    x, lg = synth.layer_inputs(cfg, 0)
    log("release %s R=%d" % (name, cfg.R))
    res = run_path(release_layer, x, lg, split=True, canary=True)
    fused = run_fused(release_layer, x, lg)
    ref = _oracle_layer(release_layer, x, lg)
    _check_values(res, ref, cfg.R)
    _check_values(fused, ref, cfg.R)
    for n in ("topk_w", "act", "out", "y"):
        assert np.array_equal(bits(res[n]), bits(fused[n])), n
    _check_chains(release_layer, x, res, range(min(cfg.R, 2)))
    log("  worst per-row relative error of y: %.2e" % float(rel_err_rows(res["y"], ref["y"]).max()))


def test_release_planted_rows_keep_class(release_layer):
    cfg = synth.CONFIGS["sixteen_random"]
    x, lg = synth.layer_inputs(cfg, 0, plant=True)
    _, (nr, _), (ir, _) = synth.plant_nan_inf(cfg.seed, 0, synth.activations(cfg.seed, 0, cfg.R, cfg.H))
    rows = [nr, ir]
    ids, _ = oracle.route(lg[rows], cfg.k)
    ex = {int(e): release_layer.host_expert(int(e)) for e in np.unique(ids)}
    ref = oracle.layer(x[rows], lg[rows], ex, cfg.H, cfg.I, cfg.E, cfg.k)
    for res in (run_path(release_layer, x, lg, canary=True), run_fused(release_layer, x, lg)):
        for name in ("act", "out", "y"):
            assert same_class(res[name][rows], ref[name]), name
            assert not np.all(np.isfinite(ref[name])), name   # the plants do reach every stage


# ---------------------------------------------------------- largest E and k
MAXED = dataclasses.replace(TINY, name="maxed", H=128, I=64, E=1024, k=16, seed=1201, weight_seed=1201)


@pytest.fixture(scope="module")
def maxed_layer():
    log("materialising 1024 small experts")
    return DeviceLayer(MAXED, 0)


@pytest.mark.parametrize("R", [1, 5, 64, 70])
def test_largest_experts_and_topk(maxed_layer, R):
    """E = 1024 and k = 16 (the ABI's limits), H = 128 (leaves 4-7 of gate/up hold
    no group and contribute +0), through both the single-workgroup (R <= 64) and
    the block routing (R > 64); the two-call path gives the same bits and
    publishes the same plan (R = 64: 1024 entries, the most that the routing
    inside the gate/up launch holds)."""
    log("maxed R=%d" % R)
    x = synth.activations(MAXED.seed, R, R, MAXED.H)
    lg = synth.logits(MAXED.seed, R, R, MAXED.E)
    res = run_path(maxed_layer, x, lg, split=True, canary=True)
    ref = _oracle_layer(maxed_layer, x, lg)
    _check_values(res, ref, R)
    _check_chains(maxed_layer, x, res, range(min(R, 3)))
    fused = run_fused(maxed_layer, x, lg)
    for n in ("topk_w", "act", "out", "y"):
        assert np.array_equal(bits(res[n]), bits(fused[n])), n
    assert np.array_equal(res["topk_id"], fused["topk_id"])
    pa, pb = read_plan(maxed_layer.d, R, res["ws"]), read_plan(maxed_layer.d, R, fused["ws"])
    for n in ("n_gu", "n_dn", "count", "offset", "entry", "gu", "dn"):
        assert np.array_equal(pa[n], pb[n]), n


@pytest.mark.parametrize("R", [1, 5, 16])
def test_tiny_general_scales(R):
    """Scale bytes over every finite E4M3FN value (negative, zero, subnormal,
    non-power-of-two) in part of the groups: values within the tolerance of the
    float64 oracle, g and u bit-equal to the fp32 replay."""
    from gpu_helpers import HostLayer
    experts = {e: synth.expert_mixed(TINY.weight_seed, 0, e, TINY.H, TINY.I, TINY.emin, TINY.emax)
               for e in range(TINY.E)}
    layer = HostLayer(TINY, experts)
    log("tiny general scales R=%d" % R)
    x = synth.activations(TINY.seed, 600 + R, R, TINY.H)
    lg = synth.logits(TINY.seed, 600 + R, R, TINY.E)
    res = run_path(layer, x, lg, split=True, canary=True)
    ref = _oracle_layer(layer, x, lg)
    _check_values(res, ref, R)
    _check_chains(layer, x, res, range(R))
    # the two-call path (down + combine in one launch at these sizes): same bits
    fused = run_fused(layer, x, lg)
    for name in ("act", "out", "y"):
        assert np.array_equal(bits(fused[name]), bits(res[name])), name
