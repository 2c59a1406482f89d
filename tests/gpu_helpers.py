"""Helpers for the GPU tests: device layers from the seeded generator and one call
that runs route -> gate/up -> down -> combine through the C ABI."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth
from fp4_routed_expert_xp_amd import xp


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class DeviceLayer:
    """Packed weights of one synthetic layer on the GPU (only the experts asked for)."""

    def __init__(self, cfg: synth.Config, layer: int = 0, experts=None, seed=None):
        self.cfg = cfg
        self.layer = layer
        self.d = xp.dims(cfg.H, cfg.I, cfg.E, cfg.k)
        ids = range(cfg.E) if experts is None else sorted(set(int(e) for e in experts))
        wseed = cfg.weight_seed if seed is None else seed
        self.packed = {}
        for e in ids:
            plain = synth.device_expert(wseed, layer, e, cfg.H, cfg.I, cfg.emin, cfg.emax)
            self.packed[e] = xp.pack_expert(plain)
            del plain
        self.table = xp.expert_table(cfg.E, self.packed)
        torch.cuda.synchronize()

    def host_expert(self, e: int) -> dict:
        return synth.layer_expert(self.cfg, self.layer, e)


class HostLayer:
    """A layer built from host experts (plain layout), packed on the GPU: for
    weights the device generator does not draw, such as general E4M3 scales."""

    def __init__(self, cfg: synth.Config, experts: dict):
        self.cfg = cfg
        self.d = xp.dims(cfg.H, cfg.I, cfg.E, cfg.k)
        self.host = experts
        self.packed = {e: xp.pack_expert({n: to_dev(a) for n, a in ex.items()}) for e, ex in experts.items()}
        self.table = xp.expert_table(cfg.E, self.packed)
        torch.cuda.synchronize()

    def host_expert(self, e: int) -> dict:
        return self.host[e]


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_path(layer: DeviceLayer, x_bits: np.ndarray, logits: np.ndarray, split: bool = False,
             canary: bool = False) -> dict:
    """Run the whole path for R rows; returns host numpy arrays (float32 as float32)."""
    d = layer.d
    R = x_bits.shape[0]
    k, H, I = d.top_k, d.hidden, d.inter
    x = to_dev(x_bits)
    lg = to_dev(logits.astype(np.float32))
    ws = torch.zeros(max(xp.xp_workspace_bytes(d, R), 256), dtype=torch.uint8, device="cuda")
    fill = float("nan") if canary else 0.0
    topk_id = torch.full((R, k), -1, dtype=torch.int32, device="cuda")
    topk_w = torch.full((R, k), fill, dtype=torch.float32, device="cuda")
    act = torch.full((R, k, I), fill, dtype=torch.float32, device="cuda")
    out = torch.full((R, k, H), fill, dtype=torch.float32, device="cuda")
    y = torch.full((R, H), fill, dtype=torch.float32, device="cuda")
    xp.xp_route_bucket(d, R, lg, topk_id, topk_w, ws)
    res = {}
    if split:
        g = torch.full((R, k, I), fill, dtype=torch.float32, device="cuda")
        u = torch.full((R, k, I), fill, dtype=torch.float32, device="cuda")
        xp.xp_gateup_rows_split(d, R, x, layer.table, ws, g, u)
        res["g"], res["u"] = g, u
    xp.xp_gateup_rows(d, R, x, layer.table, ws, act)
    xp.xp_down_rows(d, R, act, layer.table, ws, out)
    xp.xp_combine(d, R, out, topk_w, y)
    torch.cuda.synchronize()
    res.update(topk_id=topk_id, topk_w=topk_w, act=act, out=out, y=y, ws=ws)
    return {kk: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for kk, v in res.items()}


def read_plan(d: xp.xp_dims, rows: int, ws: np.ndarray) -> dict:
    """The plan fields of a workspace (host copy), by the documented layout."""
    off = xp.xp_workspace_layout(d, rows)
    b = ws.view(np.uint8)
    i32 = lambda o, n: b[o:o + 4 * n].view(np.int32).copy()
    hdr = i32(off[0], 2)
    E, nk = d.n_experts, rows * d.top_k
    return dict(n_gu=int(hdr[0]), n_dn=int(hdr[1]), count=i32(off[1], E), offset=i32(off[2], E + 1),
                entry=i32(off[3], nk), gu=i32(off[4], 4 * int(hdr[0])).reshape(-1, 4),
                dn=i32(off[5], 4 * int(hdr[1])).reshape(-1, 4))


def rel_err_rows(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per row: max |gpu - ref| / max |ref| over the oracle's finite entries (NaN if none)."""
    R = ref.shape[0]
    g = gpu.reshape(R, -1).astype(np.float64)
    r = ref.reshape(R, -1).astype(np.float64)
    out = np.empty(R)
    for i in range(R):
        m = np.isfinite(r[i])
        if not m.any():
            out[i] = 0.0
            continue
        scale = np.max(np.abs(r[i][m]))
        out[i] = np.max(np.abs(g[i][m] - r[i][m])) / scale if scale > 0 else np.max(np.abs(g[i][m]))
    return out


def same_class(gpu: np.ndarray, ref: np.ndarray) -> bool:
    """Non-finite entries agree in class: NaN <-> NaN, +Inf <-> +Inf, -Inf <-> -Inf."""
    g = gpu.astype(np.float64)
    r = ref.astype(np.float64)
    nr = ~np.isfinite(r)
    ng = ~np.isfinite(g)
    if not np.array_equal(nr, ng):
        return False
    return np.array_equal(np.isnan(g[nr]), np.isnan(r[nr])) and \
        np.array_equal(np.sign(g[nr & ~np.isnan(r)]), np.sign(r[nr & ~np.isnan(r)]))


def bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def run_fused(layer: DeviceLayer, x_bits: np.ndarray, logits: np.ndarray, repeat_down: int = 1) -> dict:
    """The two-launch path: xp_route_gateup then xp_down_combine (optionally repeated on one plan)."""
    d = layer.d
    R = x_bits.shape[0]
    k, H, I = d.top_k, d.hidden, d.inter
    x = to_dev(x_bits)
    lg = to_dev(logits.astype(np.float32))
    ws = torch.zeros(max(xp.xp_workspace_bytes(d, R), 256), dtype=torch.uint8, device="cuda")
    nan = float("nan")
    topk_id = torch.full((R, k), -1, dtype=torch.int32, device="cuda")
    topk_w = torch.full((R, k), nan, dtype=torch.float32, device="cuda")
    act = torch.full((R, k, I), nan, dtype=torch.float32, device="cuda")
    out = torch.full((R, k, H), nan, dtype=torch.float32, device="cuda")
    y = torch.full((R, H), nan, dtype=torch.float32, device="cuda")
    xp.xp_route_gateup(d, R, lg, x, layer.table, topk_id, topk_w, ws, act)
    ys = []
    for _ in range(repeat_down):
        y.fill_(nan)
        xp.xp_down_combine(d, R, act, layer.table, topk_w, ws, out, y)
        ys.append(y.clone())
    torch.cuda.synchronize()
    res = dict(topk_id=topk_id, topk_w=topk_w, act=act, out=out, y=y, ws=ws)
    res = {kk: v.cpu().numpy() for kk, v in res.items()}
    res["y_each"] = [t.cpu().numpy() for t in ys]
    return res
