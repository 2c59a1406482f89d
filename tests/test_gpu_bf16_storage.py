"""GPU: the bf16-storage variants (xp_gateup_rows_act16, xp_down_rows_act16, xp_combine_y16).

Each variant is its fp32 call followed by one round-to-nearest-even, so the checks are
bit for bit against the fp32 calls: act16 = bf16(act), down over act16 = down over act16
widened, y16 = bf16(y). Against the float64 oracle (act rounded to bf16 before down) the
values meet the per-row tolerance below: where act's fp32 and float64 values round to
neighbouring bf16 values the stored element moves by one bf16 step. A row's bits do not
depend on the other rows of the launch (NaN and +Inf planted).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from fp4_routed_expert_xp_amd import xp

from gpu_helpers import DeviceLayer, log, rel_err_rows, to_dev

pytestmark = pytest.mark.gpu

# The fp32 path's 1e-3, plus one bf16 step (at most 2^-7 of the element) where act's fp32
# and float64 values round to neighbouring bf16 values: a single product can carry the
# row's largest output. y16 adds its own rounding, 2^-9 relative.
TOL = 1e-3 + 2.0 ** -7
TOL_Y16 = TOL + 2.0 ** -9


def widen(bits16: np.ndarray) -> np.ndarray:
    return (np.asarray(bits16).view(np.uint16).astype(np.uint32) << 16).view(np.float32)


def run_both(layer: DeviceLayer, x_bits, logits) -> dict:
    """The fp32 calls and the bf16-storage calls on one plan."""
    d = layer.d
    R = x_bits.shape[0]
    k, H, I = d.top_k, d.hidden, d.inter
    dev = dict(device="cuda")
    x = to_dev(x_bits)
    lg = to_dev(logits.astype(np.float32))
    ws = torch.zeros(max(xp.xp_workspace_bytes(d, R), 256), dtype=torch.uint8, **dev)
    topk_id = torch.full((R, k), -1, dtype=torch.int32, **dev)
    topk_w = torch.full((R, k), float("nan"), dtype=torch.float32, **dev)
    act = torch.full((R, k, I), float("nan"), dtype=torch.float32, **dev)
    act16 = torch.full((R, k, I), -1, dtype=torch.int16, **dev)
    out = torch.full((R, k, H), float("nan"), dtype=torch.float32, **dev)
    out16 = torch.full((R, k, H), float("nan"), dtype=torch.float32, **dev)
    out_w = torch.full((R, k, H), float("nan"), dtype=torch.float32, **dev)
    y = torch.full((R, H), float("nan"), dtype=torch.float32, **dev)
    y16 = torch.full((R, H), -1, dtype=torch.int16, **dev)
    xp.xp_route_bucket(d, R, lg, topk_id, topk_w, ws)
    xp.xp_gateup_rows(d, R, x, layer.table, ws, act)
    xp.xp_gateup_rows_act16(d, R, x, layer.table, ws, act16)
    xp.xp_down_rows(d, R, act, layer.table, ws, out)
    xp.xp_down_rows_act16(d, R, act16, layer.table, ws, out16)
    widened = (act16.to(torch.int32) << 16).view(torch.float32).contiguous()
    xp.xp_down_rows(d, R, widened, layer.table, ws, out_w)
    xp.xp_combine(d, R, out16, topk_w, y)
    xp.xp_combine_y16(d, R, out16, topk_w, y16)
    torch.cuda.synchronize()
    res = dict(topk_id=topk_id, topk_w=topk_w, act=act, act16=act16, out=out, out16=out16, out_w=out_w,
               y=y, y16=y16)
    return {kk: v.cpu().numpy() for kk, v in res.items()}


def rne(f32: np.ndarray) -> np.ndarray:
    return synth.f32_to_bf16_bits(f32).view(np.int16)


def check_bits(res):
    assert np.array_equal(res["act16"], rne(res["act"]))
    assert np.array_equal(res["out16"].view(np.uint32), res["out_w"].view(np.uint32))
    assert np.array_equal(res["y16"], rne(res["y"]))


@pytest.fixture(scope="module")
def tiny_layer():
    return DeviceLayer(synth.CONFIGS["tiny"], 0)


@pytest.mark.parametrize("R", [1, 4, 9, 70])
def test_tiny_bf16_storage(tiny_layer, R):
    cfg = tiny_layer.cfg
    x = synth.activations(cfg.seed, 200 + R, R, cfg.H)
    lg = synth.logits(cfg.seed, 200 + R, R, cfg.E)
    res = run_both(tiny_layer, x, lg)
    check_bits(res)
    ex = {e: tiny_layer.host_expert(e) for e in range(cfg.E)}
    ref = oracle.layer(x, lg, ex, cfg.H, cfg.I, cfg.E, cfg.k, act_bf16=True)
    assert np.array_equal(res["topk_id"], ref["topk_id"])
    measured = {}
    for name, got, tol in (("act", widen(res["act16"]), TOL), ("out", res["out16"], TOL),
                           ("y", widen(res["y16"]), TOL_Y16)):
        err = rel_err_rows(got, ref[name])
        assert np.all(err <= tol), (name, float(err.max()))
        measured[name] = float(err.max())
    log("tiny R=%d: bf16 storage within tolerance (measured max per-row error act %.2e, out %.2e, y16 %.2e "
        "against bounds %.2e / %.2e / %.2e), bits equal to the fp32 calls rounded"
        % (R, measured["act"], measured["out"], measured["y"], TOL, TOL, TOL_Y16))


@pytest.fixture(scope="module")
def release_layer():
    cfg = synth.CONFIGS["sixteen_random"]
    x, lg = synth.layer_inputs(cfg, 0)
    ids, _ = oracle.route(lg, cfg.k)
    return DeviceLayer(cfg, 0, experts=np.unique(ids))


def test_release_width_rows_alone(release_layer):
    """Sixteen random rows at release widths (NaN and +Inf planted in two rows):
    the bit relations to the fp32 calls hold, and every row's act16, out and y16
    equal that row launched alone."""
    cfg = release_layer.cfg
    x, lg = synth.layer_inputs(cfg, 0)
    full = run_both(release_layer, x, lg)
    check_bits(full)
    ex = {int(e): release_layer.host_expert(int(e)) for e in release_layer.packed}
    ref = oracle.layer(x, lg, ex, cfg.H, cfg.I, cfg.E, cfg.k, act_bf16=True)
    measured = {}
    for name, got, tol in (("act", widen(full["act16"]), TOL), ("out", full["out16"], TOL),
                           ("y", widen(full["y16"]), TOL_Y16)):
        err = rel_err_rows(got, ref[name])
        assert np.all(err <= tol), (name, float(err.max()))
        measured[name] = float(err.max())
    log("release 16 rows: measured max per-row error against the float64 oracle with bf16 act: act %.2e, "
        "out %.2e, y16 %.2e" % (measured["act"], measured["out"], measured["y"]))
    for r in (0, 3, 7, 15):
        one = run_both(release_layer, x[r:r + 1], lg[r:r + 1])
        for name in ("act16", "out16", "y16"):
            assert np.array_equal(full[name][r:r + 1].view(np.uint16), one[name].view(np.uint16)), (r, name)
