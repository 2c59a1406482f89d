"""GPU: gate/up over E4M3FN-coded activations with one E8M0 scale per 32
(xp_gateup_rows_coded).

- act is bit-equal to xp_gateup_rows on bf16 activations holding the same
  values (the coded value e4m3(code) * 2^(scale - 127) is formed exactly and
  enters the same chain);
- act, and out and y after the fp32 down and combine, are within the per-row
  tolerance (1e-3) of the float64 oracle's coded layer (oracle.layer_coded);
- each row's act equals its solo launch bit for bit, and a NaN scale byte stays
  in its row.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from fp4_routed_expert_xp_amd import xp

from gpu_helpers import DeviceLayer, bits, log, rel_err_rows, same_class, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3
TINY = synth.CONFIGS["tiny"]


def run_coded(layer, codes, scales, lg, also_bf16=True):
    """Route, coded gate/up, down, combine; and gate/up on the same values as bf16."""
    d = layer.d
    R = codes.shape[0]
    k, H, I = d.top_k, d.hidden, d.inter
    ws = torch.zeros(max(xp.xp_workspace_bytes(d, R), 256), dtype=torch.uint8, device="cuda")
    nan = float("nan")
    ids = torch.full((R, k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((R, k), nan, dtype=torch.float32, device="cuda")
    act = torch.full((R, k, I), nan, dtype=torch.float32, device="cuda")
    out = torch.full((R, k, H), nan, dtype=torch.float32, device="cuda")
    y = torch.full((R, H), nan, dtype=torch.float32, device="cuda")
    xp.xp_route_bucket(d, R, to_dev(lg.astype(np.float32)), ids, w, ws)
    xp.xp_gateup_rows_coded(d, R, to_dev(codes), to_dev(scales), layer.table, ws, act)
    xp.xp_down_rows(d, R, act, layer.table, ws, out)
    xp.xp_combine(d, R, out, w, y)
    res = dict(topk_id=ids, act=act, out=out, y=y)
    if also_bf16:
        xf = oracle.dequant_coded(codes, scales).astype(np.float32)
        xb = synth.f32_to_bf16_bits(xf)
        act_b = torch.full((R, k, I), nan, dtype=torch.float32, device="cuda")
        xp.xp_gateup_rows(d, R, to_dev(xb), layer.table, ws, act_b)
        res["act_bf16"] = act_b
    torch.cuda.synchronize()
    return {n: v.cpu().numpy() for n, v in res.items()}


def _oracle(layer, codes, scales, lg):
    cfg = layer.cfg
    ids, _ = oracle.route(lg, cfg.k)
    ex = {int(e): layer.host_expert(int(e)) for e in np.unique(ids)}
    return oracle.layer_coded(codes, scales, lg, ex, cfg.H, cfg.I, cfg.E, cfg.k)


def _check(res, ref):
    assert np.array_equal(res["topk_id"], ref["topk_id"])
    for n in ("act", "out", "y"):
        err = rel_err_rows(res[n], ref[n])
        assert np.all(err <= TOL), (n, err)
        assert same_class(res[n], ref[n]), n
    return max(float(rel_err_rows(res[n], ref[n]).max()) for n in ("act", "out", "y"))


@pytest.fixture(scope="module")
def tiny_layer():
    return DeviceLayer(TINY, 0)


@pytest.fixture(scope="module")
def release_layer():
    log("materialising release-width layer 0 (256 experts)")
    return DeviceLayer(synth.CONFIGS["one_row"], 0)


@pytest.mark.parametrize("R", [1, 3, 4, 9, 16, 65])
def test_tiny_coded_matches_bf16_path_and_oracle(tiny_layer, R):
    codes, scales = synth.coded_activations(TINY.seed + 60, R, R, TINY.H)
    lg = synth.logits(TINY.seed + 60, R, R, TINY.E)
    res = run_coded(tiny_layer, codes, scales, lg)
    assert np.array_equal(bits(res["act"]), bits(res["act_bf16"]))
    worst = _check(res, _oracle(tiny_layer, codes, scales, lg))
    log("coded tiny R=%d: worst per-row relative error %.2e" % (R, worst))


@pytest.mark.parametrize("name", ["one_row", "four_same", "sixteen_random"])
def test_release_coded(release_layer, name):
    cfg = synth.CONFIGS[name]
    _, lg = synth.layer_inputs(cfg, 0)
    codes, scales = synth.coded_activations(cfg.seed + 60, 0, cfg.R, cfg.H)
    log("coded release %s R=%d" % (name, cfg.R))
    res = run_coded(release_layer, codes, scales, lg)
    assert np.array_equal(bits(res["act"]), bits(res["act_bf16"]))
    worst = _check(res, _oracle(release_layer, codes, scales, lg))
    log("  worst per-row relative error %.2e" % worst)


@pytest.mark.parametrize("routing", ["same", "random"])
def test_coded_rows_equal_their_solo_launch(tiny_layer, routing):
    R = 9
    codes, scales = synth.coded_activations(TINY.seed + 61, R, R, TINY.H)
    lg = (synth.logits_same if routing == "same" else synth.logits)(TINY.seed + 61, R, R, TINY.E)
    batch = run_coded(tiny_layer, codes, scales, lg, also_bf16=False)
    for r in range(R):
        solo = run_coded(tiny_layer, codes[r:r + 1], scales[r:r + 1], lg[r:r + 1], also_bf16=False)
        for n in ("act", "out", "y"):
            assert np.array_equal(bits(batch[n][r]), bits(solo[n][0])), (routing, r, n)


def test_nan_scale_stays_in_its_row(tiny_layer):
    R = 4
    codes, scales = synth.coded_activations(TINY.seed + 62, R, R, TINY.H)
    scales = scales.copy()
    scales[2, 3] = 0xFF
    lg = synth.logits_same(TINY.seed + 62, R, R, TINY.E)
    res = run_coded(tiny_layer, codes, scales, lg, also_bf16=False)
    ref = _oracle(tiny_layer, codes, scales, lg)
    for n in ("act", "out", "y"):
        assert same_class(res[n], ref[n]), n
    assert np.all(np.isnan(res["act"][2])) and np.all(np.isfinite(res["act"][[0, 1, 3]]))
