"""GPU: the two-launch path (xp_route_gateup, xp_down_combine) against the four calls.

Both paths run the same per-row arithmetic, so every output must be bit-equal,
the published plan must be the same, and repeated down+combine launches on one
plan must keep giving the same y. xp_route_gateup routes inside the gate/up
launch for one row (gateup_one_row_kernel) and for 2..64 rows whose gate/up
grid is at most 1024 workgroups (route_gateup_rows_kernel), and otherwise runs
the routing launch first. xp_down_combine runs one of three forms: one
row with top-k up to 8 in down_combine_one_row_kernel, at most 64 (row, slot)
entries in down_combine_rows_kernel, and more entries as the two launches
(down, then combine); each form is covered below, and the two-call path is
also probed row by row against its own solo launches at release width."""
import numpy as np
import pytest

import synth
from fp4_routed_expert_xp_amd import xp

from gpu_helpers import DeviceLayer, bits, log, read_plan, run_fused, run_path

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny_layer():
    return DeviceLayer(synth.CONFIGS["tiny"], 0)


@pytest.fixture(scope="module")
def release_layer():
    log("materialising release-width layer 0 (256 experts)")
    return DeviceLayer(synth.CONFIGS["one_row"], 0)


def _compare(layer, x, lg, tag):
    a = run_path(layer, x, lg)
    b = run_fused(layer, x, lg, repeat_down=3)
    assert np.array_equal(a["topk_id"], b["topk_id"]), tag
    for n in ("topk_w", "act", "out", "y"):
        assert np.array_equal(bits(a[n]), bits(b[n])), (tag, n)
    for yy in b["y_each"]:
        assert np.array_equal(bits(yy), bits(a["y"])), (tag, "repeat")
    pa, pb = read_plan(layer.d, x.shape[0], a["ws"]), read_plan(layer.d, x.shape[0], b["ws"])
    for n in ("count", "offset", "entry", "gu", "dn"):
        assert np.array_equal(pa[n], pb[n]), (tag, n)
    assert (pa["n_gu"], pa["n_dn"]) == (pb["n_gu"], pb["n_dn"]), tag


@pytest.mark.parametrize("R", [1, 2, 4, 5, 16, 64, 65, 100])
def test_fused_equals_four_calls_tiny(tiny_layer, R):
    cfg = tiny_layer.cfg
    x = synth.activations(cfg.seed + 5, R, R, cfg.H)
    lg = synth.logits(cfg.seed + 5, R, R, cfg.E)
    if R >= 2:
        x, _, _ = synth.plant_nan_inf(cfg.seed, R, x)
    _compare(tiny_layer, x, lg, "tiny R=%d" % R)


@pytest.mark.parametrize("name", ["one_row", "four_same", "sixteen_random"])
def test_fused_equals_four_calls_release(release_layer, name):
    cfg = synth.CONFIGS[name]
    x, lg = synth.layer_inputs(cfg, 0)
    log("fused %s" % name)
    _compare(release_layer, x, lg, name)


@pytest.mark.parametrize("tiers", [((4,), (4,)), ((2, 4, 8), (2, 4, 8))])
def test_fused_other_tiers(release_layer, tiers):
    cfg = synth.CONFIGS["sixteen_random"]
    x = synth.activations(cfg.seed, 7, 16, cfg.H)
    lg = synth.logits_same(cfg.seed, 7, 16, cfg.E)
    lg[8:] = synth.logits(cfg.seed, 7, 8, cfg.E)
    xp.xp_set_tiers(list(tiers[0]), list(tiers[1]))
    try:
        _compare(release_layer, x, lg, "tiers %s" % (tiers,))
    finally:
        xp.xp_set_tiers(None, None)


def test_fused_probe_tiny(tiny_layer):
    cfg = tiny_layer.cfg
    for R in (3, 9, 16):
        x = synth.activations(cfg.seed + 9, R, R, cfg.H)
        lg = synth.logits_same(cfg.seed + 9, R, R, cfg.E)
        batch = run_fused(tiny_layer, x, lg)
        for r in range(R):
            solo = run_fused(tiny_layer, x[r:r + 1], lg[r:r + 1])
            for n in ("act", "out", "y"):
                assert np.array_equal(bits(batch[n][r]), bits(solo[n][0])), (R, r, n)


@pytest.mark.parametrize("k", [1, 3, 4, 5, 8, 9])
def test_fused_one_row_every_top_k(k):
    """One row: xp_down_combine runs down and combine in down_combine_one_row_kernel
    for top-k up to 8 (passes 4 per row-group of lanes, the last group partly idle
    when k is not a multiple of 4) and in down_combine_rows_kernel above 8 (one
    row's k entries are at most 64); every case bit-equal to the four calls.
    Width 256 x 192 (three 64-column tiles, six groups per leaf walk)."""
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], name="tiny_k%d" % k, H=256, I=192, E=12, k=k,
                              seed=1200 + k, weight_seed=1200)
    layer = DeviceLayer(cfg, 0)
    x = synth.activations(cfg.seed, 1, 1, cfg.H)
    lg = synth.logits(cfg.seed, 1, 1, cfg.E)
    _compare(layer, x, lg, "one row k=%d" % k)


@pytest.mark.parametrize("dn", [(2, 4, 8), (3, 5, 7), (8,)])
def test_fused_few_entries_large_passes(tiny_layer, dn):
    """At most 64 (row, slot) entries: xp_down_combine's one-launch kernel with
    down passes of 5 to 8 rows (a wave running the largest size among its rows
    of lanes, shorter passes padded), same-expert and mixed routing; bit-equal
    to the four calls."""
    cfg = tiny_layer.cfg
    xp.xp_set_tiers([2, 4, 6, 8], list(dn))
    try:
        for R in (8, 13, 32):
            x = synth.activations(cfg.seed + 11, R, R, cfg.H)
            lg = synth.logits_same(cfg.seed + 11, R, R, cfg.E)
            lg[R // 2:] = synth.logits(cfg.seed + 12, R, R - R // 2, cfg.E)
            _compare(tiny_layer, x, lg, "dn %s R=%d" % (dn, R))
    finally:
        xp.xp_set_tiers(None, None)


PROBE_FUSED_ROWS = [2, 3, 5, 7, 8]


@pytest.mark.parametrize("routing", ["same", "disjoint", "random"])
def test_fused_probe_release(release_layer, routing):
    """The headline two-call path at release width, at the row counts whose down
    passes take every form of down_combine_rows_kernel (2 to 8 rows, 16 to 64
    entries): each row of the batch bit-equal to the same row launched alone on
    the two-call path, and the batch bit-equal to the four calls."""
    cfg = release_layer.cfg
    for R in PROBE_FUSED_ROWS:
        x = synth.activations(cfg.seed + 31, R, R, cfg.H)
        if routing == "same":
            lg = synth.logits_same(cfg.seed + 31, R, R, cfg.E)
        elif routing == "disjoint":
            lg = synth.logits_disjoint(R, cfg.E, cfg.k)
        else:
            lg = synth.logits(cfg.seed + 31, R, R, cfg.E)
        x, _, _ = synth.plant_nan_inf(cfg.seed + 31, R, x)
        log("fused probe release R=%d %s" % (R, routing))
        batch = run_fused(release_layer, x, lg)
        four = run_path(release_layer, x, lg)
        for n in ("act", "out", "y"):
            assert np.array_equal(bits(batch[n]), bits(four[n])), (R, routing, n)
        for r in range(R):
            solo = run_fused(release_layer, x[r:r + 1], lg[r:r + 1])
            for n in ("act", "out", "y"):
                assert np.array_equal(bits(batch[n][r]), bits(solo[n][0])), (R, routing, r, n)


@pytest.mark.parametrize("dn", [(3, 5, 7), (8,)])
def test_fused_large_passes_long_leaf_walk(dn):
    """down_combine_rows_kernel with passes of 3 to 8 rows on a layer whose down
    K (intermediate 1024: 32 groups, four per leaf) is longer than every pass
    size's weight ring, so each ring refills inside the leaf walk; bit-equal to
    the four calls under same-expert and mixed routing."""
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], name="tiny_i1024", H=256, I=1024, E=8, k=2,
                              seed=1300, weight_seed=1300)
    layer = DeviceLayer(cfg, 0)
    xp.xp_set_tiers([2, 4, 6, 8], list(dn))
    try:
        for R in (3, 8, 13, 32):
            x = synth.activations(cfg.seed, R, R, cfg.H)
            lg = synth.logits_same(cfg.seed, R, R, cfg.E)
            lg[R // 2:] = synth.logits(cfg.seed + 1, R, R - R // 2, cfg.E)
            _compare(layer, x, lg, "I=1024 dn %s R=%d" % (dn, R))
    finally:
        xp.xp_set_tiers(None, None)
