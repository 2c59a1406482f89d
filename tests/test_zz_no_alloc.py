"""GPU: xp_decode_static, the two-call decode path with its plan in the
library's own device array (no workspace, no allocation), against
xp_route_gateup + xp_down_combine with a caller workspace: every output bit
for bit, on two calls in a row (the second with fewer rows, so the array
keeps the first call's larger plan underneath), at tiny and release widths."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from fp4_routed_expert_xp_amd import xp

from gpu_helpers import DeviceLayer, bits, log, run_fused, to_dev

pytestmark = pytest.mark.gpu

STATIC_BYTES = 1 << 20


def run_static(layer, x_bits, logits):
    d = layer.d
    R = x_bits.shape[0]
    k, H, I = d.top_k, d.hidden, d.inter
    nan = float("nan")
    topk_id = torch.full((R, k), -1, dtype=torch.int32, device="cuda")
    topk_w = torch.full((R, k), nan, dtype=torch.float32, device="cuda")
    act = torch.full((R, k, I), nan, dtype=torch.float32, device="cuda")
    out = torch.full((R, k, H), nan, dtype=torch.float32, device="cuda")
    y = torch.full((R, H), nan, dtype=torch.float32, device="cuda")
    xp.xp_decode_static(d, R, to_dev(logits.astype(np.float32)), to_dev(x_bits), layer.table, topk_id, topk_w,
                        act, out, y)
    torch.cuda.synchronize()
    return {n: v.cpu().numpy() for n, v in
            dict(topk_id=topk_id, topk_w=topk_w, act=act, out=out, y=y).items()}


def _same(a, b, tag):
    assert np.array_equal(a["topk_id"], b["topk_id"]), tag
    for n in ("topk_w", "act", "out", "y"):
        assert np.array_equal(bits(a[n]), bits(b[n])), (tag, n)


@pytest.mark.parametrize("cfg_name,rows", [("tiny", (16, 3)), ("one_row", (8, 1))])
def test_static_equals_two_calls_twice(cfg_name, rows):
    cfg = synth.CONFIGS[cfg_name]
    layer = DeviceLayer(cfg, 0)
    for i, R in enumerate(rows):
        log("static %s call %d R=%d" % (cfg_name, i, R))
        x = synth.activations(cfg.seed + 41 + i, R, R, cfg.H)
        lg = synth.logits(cfg.seed + 41 + i, R, R, cfg.E)
        if R >= 2:
            x, _, _ = synth.plant_nan_inf(cfg.seed + 41, R, x)
        _same(run_static(layer, x, lg), run_fused(layer, x, lg), "%s R=%d" % (cfg_name, R))


def test_static_refuses_a_plan_larger_than_its_array():
    d = xp.dims(4096, 2048, 256, 8)
    big = 1
    while xp.xp_workspace_bytes(d, big) <= STATIC_BYTES:
        big += 64
    P = ctypes.c_void_p(0x1000)
    L = xp.lib()
    assert L.xp_decode_static(ctypes.byref(d), big, P, P, P, P, P, P, P, P, None) == xp.XP_ERR_WORKSPACE
    assert L.xp_decode_static(ctypes.byref(d), 0, None, None, None, None, None, None, None, None, None) == xp.XP_OK
    assert L.xp_decode_static(ctypes.byref(d), 4, P, None, P, P, P, P, P, P, None) == xp.XP_ERR_NULL
