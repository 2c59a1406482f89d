"""GPU: the batch-invariance probe.

A launch's act, out and combine output y must equal, bit for bit (NaN payloads
included), the same row launched alone, for same, disjoint and random routing,
finite and with NaN and +Inf planted, at rows 1, 2, 3, 4, 5, 7, 8, 9 and 16:
54 cases. [#2983, "Receipt": the equality probe] Every row count from 2 to 16
is also run (same/disjoint/mixed), and alternative pass-size sets must give
the same bits. The ground truth is the solo launch, which runs the one-row
pass for every expert.
"""
import numpy as np
import pytest

import synth
from fp4_routed_expert_xp_amd import xp

from gpu_helpers import DeviceLayer, bits, log, run_path

pytestmark = pytest.mark.gpu

PROBE_ROWS = [1, 2, 3, 4, 5, 7, 8, 9, 16]
ROUTINGS = ["same", "disjoint", "random"]


def _inputs(cfg, R, routing, planted, salt=0):
    x = synth.activations(cfg.seed + 17 + salt, R, R, cfg.H)
    if routing == "same":
        lg = synth.logits_same(cfg.seed + 17 + salt, R, R, cfg.E)
    elif routing == "disjoint":
        lg = synth.logits_disjoint(R, cfg.E, cfg.k)
    elif routing == "random":
        lg = synth.logits(cfg.seed + 17 + salt, R, R, cfg.E)
    else:  # mixed: half the rows share row 0's logits
        lg = synth.logits(cfg.seed + 17 + salt, R, R, cfg.E)
        lg[: (R + 1) // 2] = lg[0]
    if planted and R >= 2:
        x, _, _ = synth.plant_nan_inf(cfg.seed + salt, R, x)
    return x, lg


def _probe(layer, x, lg):
    """Number of rows whose act/out/y differ from their solo launch."""
    batch = run_path(layer, x, lg)
    bad = 0
    for r in range(x.shape[0]):
        solo = run_path(layer, x[r:r + 1], lg[r:r + 1])
        same = all(np.array_equal(bits(batch[n][r]), bits(solo[n][0])) for n in ("act", "out", "y"))
        same = same and np.array_equal(batch["topk_id"][r], solo["topk_id"][0])
        bad += 0 if same else 1
    return bad


@pytest.fixture(scope="module")
def tiny_layer():
    return DeviceLayer(synth.CONFIGS["tiny"], 0)


@pytest.fixture(scope="module")
def release_layer():
    log("materialising release-width layer 0 (256 experts)")
    return DeviceLayer(synth.CONFIGS["one_row"], 0)


def _matrix(layer, tag):
    cfg = layer.cfg
    differ, cases, red = 0, 0, 0
    for R in PROBE_ROWS:
        for routing in ROUTINGS:
            for planted in (False, True):
                x, lg = _inputs(cfg, R, routing, planted)
                bad = _probe(layer, x, lg)
                log("probe %s R=%d %s %s: %d rows differ" % (tag, R, routing, "planted" if planted else "finite",
                                                               bad))
                differ += bad
                cases += 1
                red += 1 if bad else 0
    log("SUMMARY probe %s: %d cases, %d equal to their solo launches, %d differ" % (tag, cases, cases - red, red))
    return differ


def test_probe_matrix_tiny(tiny_layer):
    assert _matrix(tiny_layer, "tiny") == 0


def test_probe_matrix_release(release_layer):
    assert _matrix(release_layer, "release") == 0


def test_probe_every_row_count_tiny(tiny_layer):
    cfg = tiny_layer.cfg
    for R in range(2, 17):
        for routing in ("same", "disjoint", "mixed"):
            x, lg = _inputs(cfg, R, routing, False, salt=1)
            assert _probe(tiny_layer, x, lg) == 0, (R, routing)


@pytest.mark.parametrize("tiers", [((4,), (4,)), ((2, 4, 6, 8), (2, 4)), ((8,), (8,)), ((2, 4, 8), (2, 4, 8))])
def test_tier_sets_give_identical_bits_release(release_layer, tiers):
    cfg = release_layer.cfg
    x, lg = _inputs(cfg, 16, "mixed", True, salt=2)
    base = run_path(release_layer, x, lg)
    xp.xp_set_tiers(list(tiers[0]), list(tiers[1]))
    try:
        other = run_path(release_layer, x, lg)
    finally:
        xp.xp_set_tiers(None, None)
    for n in ("act", "out", "y"):
        assert np.array_equal(bits(base[n]), bits(other[n])), n
