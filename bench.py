#!/usr/bin/env python3
"""Bench: MoE decode rows/s and expert-weight HBM GB/s (% of peak) on one MI355X.

A step is one 40-layer round: 40 independent synthetic release-width layers
(hidden 4096, expert intermediate 2048, 256 experts, top-8), each running the
whole hot path (route + bucket, gate/up + SwiGLU, down, combine) through the C
ABI. The round is captured once as a HIP graph and replayed; all weights
(40 x 256 experts, 13,369,344 B each) are resident in HBM before timing.

The headline is the one-row workload on the two-launch path (xp_route_gateup,
xp_down_combine); every workload is also timed on the four-call path, and the
four-row same-expert and sixteen-row random workloads are extra cells on the
same line.
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE decode rows/s + expert-weight HBM GB/s (% of peak), 1–16 rows/layer"
HBM_PEAK_GBPS = 8000.0
CUS, LANES, CLOCK_GHZ = 256, 64, 2.4     # fp32 vector fma lanes per CU per clock, unpacked
CSRC = os.path.join(ROOT, "fp4_routed_expert_xp_amd", "csrc")

# HBM bytes per launch of the roofline kernel (gateup_one_row_kernel, one-row
# workload), from two rocprofv3 --pmc runs: FETCH_SIZE, then WRITE_SIZE, in KiB per
# dispatch (mean over the dispatches of that workload). Each is scaled by what the
# same counter read for a plain 2 GiB device-to-device copy: FETCH_SIZE read
# 1,048,613.5 KiB for 2,097,152 KiB fetched, WRITE_SIZE read exactly 2,097,152 KiB.
# The figure belongs to the sources the kernel is built from (their digest below);
# after any change to them the bench reports traffic as null.
TRAFFIC = dict(sources="24b08809", fetch_kib=35001.6, write_kib=66.4,
               fetch_factor=2097152 / 1048613.5, write_factor=1.0)
ROOFLINE_SOURCES = ("xp_rows.hip", "xp_pass_dev.h", "xp_common.h", "xp_route_dev.h", "xp_chain_asm.h")
# The same counters for the one-row down + combine launch (down_combine_one_row_kernel).
DOWN_TRAFFIC = dict(sources="24b08809", fetch_kib=17734.4, write_kib=144.0)
# The same for the dense FP8 projection kernel at 4096 x 4096 (grid of 256
# workgroups; mean over its launches at 1, 8 and 16 rows), tied to xp_fp8.hip.
FP8_TRAFFIC = dict(sources="15929da9", fetch_kib=8532.4, write_kib=133.3)
FP8_SOURCES = ("xp_fp8.hip", "xp_common.h")
# The same for the two prefill kernels on the 4,096-row chunk (mean over 4 seeded
# layers), tied to xp_prefill.hip and its headers.
PF_GU_TRAFFIC = dict(sources="228f5abb", fetch_kib=1654531.8, write_kib=262468.0)
PF_DN_TRAFFIC = dict(sources="228f5abb", fetch_kib=865250.3, write_kib=524458.8)
PREFILL_SOURCES = ("xp_prefill.hip", "xp_prefill_asm.h", "xp_common.h")


def csrc_digest(sources=ROOFLINE_SOURCES) -> str:
    """Digest of a kernel's sources (its .hip file and the internal headers it includes)."""
    import hashlib
    h = hashlib.sha256()
    for name in sources:
        h.update(name.encode())
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:8]


def measured_traffic(t=None, sources=ROOFLINE_SOURCES):
    """HBM bytes per launch of a roofline kernel, or None once its sources changed."""
    t = TRAFFIC if t is None else t
    if csrc_digest(sources) != t["sources"]:
        return None
    kib = t["fetch_kib"] * TRAFFIC["fetch_factor"] + t["write_kib"] * TRAFFIC["write_factor"]
    return int(round(kib * 1024))


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=40)
    ap.add_argument("--cells", default="one_row,four_same,sixteen_random,prefill,fp8_rows")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tier-sweep", action="store_true", help="skip the pass-size sweep cells")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU work budget of the oracle sample")
    return ap.parse_args()


# ---------------------------------------------------------------- weights
class Model:
    """40 layers x 256 experts of packed weights, one uint8 buffer per layer."""

    def __init__(self, cfg, layers: int):
        import torch
        import synth
        from fp4_routed_expert_xp_amd import xp
        self.cfg = cfg
        H, I, E = cfg.H, cfg.I, cfg.E
        self.expert_bytes = cfg.expert_bytes
        plain = torch.empty(E * self.expert_bytes, dtype=torch.uint8, device="cuda")
        self.buffers, self.tables = [], []
        shapes = {"gate": (I, H), "up": (I, H), "down": (H, I)}
        for l in range(layers):
            lay = synth.device_layer_plain(cfg.weight_seed, l, H, I, E, cfg.emin, cfg.emax, plain)
            stride, offs = lay["stride"], lay["offsets"]
            packed = torch.empty_like(plain)
            tab = []
            for e in range(E):
                row = []
                for m in ("gate", "up", "down"):
                    N, K = shapes[m]
                    co, cn = offs[m + "_codes"]
                    so, sn = offs[m + "_scales"]
                    b = e * stride
                    xp.xp_pack_matrix(plain[b + co:b + co + cn].view(N, K // 2), plain[b + so:b + so + sn],
                                      packed[b + co:b + co + cn], packed[b + so:b + so + sn])
                    row += [packed.data_ptr() + b + co, packed.data_ptr() + b + so]
                tab.append(row)
            self.buffers.append(packed)
            self.tables.append(torch.tensor(tab, dtype=torch.int64).cuda())
        torch.cuda.synchronize()
        del plain


def copy_bandwidth_gbps() -> float:
    import torch
    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    return 2 * n / sec / 1e9


# ------------------------------------------------------------------ cells
class Cell:
    def __init__(self, model: Model, cfg, layers: int):
        import numpy as np
        import torch
        import synth
        from fp4_routed_expert_xp_amd import xp
        self.model, self.cfg, self.layers = model, cfg, layers
        R, k, H, I, E = cfg.R, cfg.k, cfg.H, cfg.I, cfg.E
        self.d = xp.dims(H, I, E, k)
        self.x, self.logits, self.ws = [], [], []
        for l in range(layers):
            xb, lg = synth.layer_inputs(cfg, l, plant=False)
            self.x.append(torch.from_numpy(xb.view(np.int16).copy()).cuda())
            self.logits.append(torch.from_numpy(lg).cuda())
            self.ws.append(torch.zeros(xp.xp_workspace_bytes(self.d, R), dtype=torch.uint8, device="cuda"))
        self.topk_id = torch.empty((R, k), dtype=torch.int32, device="cuda")
        self.topk_w = torch.empty((R, k), dtype=torch.float32, device="cuda")
        self.act = torch.empty((R, k, I), dtype=torch.float32, device="cuda")
        self.out = torch.empty((R, k, H), dtype=torch.float32, device="cuda")
        self.y = torch.empty((R, H), dtype=torch.float32, device="cuda")
        self.act16 = torch.empty((R, k, I), dtype=torch.int16, device="cuda")
        self.y16 = torch.empty((R, H), dtype=torch.int16, device="cuda")

    def call(self, kind: str, l: int) -> None:
        """One library call of layer l."""
        from fp4_routed_expert_xp_amd import xp
        d, R, tab, ws = self.d, self.cfg.R, self.model.tables[l], self.ws[l]
        if kind == "route":
            xp.xp_route_bucket(d, R, self.logits[l], self.topk_id, self.topk_w, ws)
        elif kind == "gateup":
            xp.xp_gateup_rows(d, R, self.x[l], tab, ws, self.act)
        elif kind == "down":
            xp.xp_down_rows(d, R, self.act, tab, ws, self.out)
        elif kind == "combine":
            xp.xp_combine(d, R, self.out, self.topk_w, self.y)
        elif kind == "route_gateup":
            xp.xp_route_gateup(d, R, self.logits[l], self.x[l], tab, self.topk_id, self.topk_w, ws, self.act)
        elif kind == "down_combine":
            xp.xp_down_combine(d, R, self.act, tab, self.topk_w, ws, self.out, self.y)
        elif kind == "gateup_act16":
            xp.xp_gateup_rows_act16(d, R, self.x[l], tab, ws, self.act16)
        elif kind == "down_act16":
            xp.xp_down_rows_act16(d, R, self.act16, tab, ws, self.out)
        elif kind == "combine_y16":
            xp.xp_combine_y16(d, R, self.out, self.topk_w, self.y16)
        elif kind == "prefill_gateup":
            xp.xp_prefill_gateup(d, R, self.x[l], tab, ws, self.act)
        elif kind == "prefill_down":
            xp.xp_prefill_down(d, R, self.act, tab, ws, self.out)
        else:
            raise ValueError(kind)

    def round(self, kinds) -> None:
        for l in range(self.layers):
            for kind in kinds:
                self.call(kind, l)

    def plan_stats(self) -> dict:
        """Distinct experts and pass sizes per layer, read back from the workspaces."""
        import numpy as np
        from fp4_routed_expert_xp_amd import xp
        off = xp.xp_workspace_layout(self.d, self.cfg.R)
        E = self.cfg.E
        distinct, gu_rows, dn_rows, gu_passes, dn_passes = [], [], [], [], []
        for ws in self.ws:
            b = ws.cpu().numpy()
            hdr = b[off[0]:off[0] + 8].view(np.int32)
            cnt = b[off[1]:off[1] + 4 * E].view(np.int32)
            gu = b[off[4]:off[4] + 16 * int(hdr[0])].view(np.int32).reshape(-1, 4)
            dn = b[off[5]:off[5] + 16 * int(hdr[1])].view(np.int32).reshape(-1, 4)
            distinct.append(int((cnt > 0).sum()))
            gu_rows.append(int(gu[:, 3].sum()))     # rows computed incl. padding
            dn_rows.append(int(dn[:, 3].sum()))
            gu_passes.append(int(hdr[0]))
            dn_passes.append(int(hdr[1]))
        return dict(distinct=distinct, gu_rows=gu_rows, dn_rows=dn_rows, gu_passes=gu_passes, dn_passes=dn_passes)


def time_stream(cell: Cell) -> dict:
    """The read-only ceiling of the cell's weight stream: xp_stream_weights over
    each layer's distinct routed experts (read back from the plans in the
    workspaces), a graph of one launch per layer, timed with events on the
    launch stream; microseconds per layer and GB/s on the same unique bytes."""
    import numpy as np
    import torch
    from fp4_routed_expert_xp_amd import xp
    off = xp.xp_workspace_layout(cell.d, cell.cfg.R)
    E = cell.cfg.E
    ids, nbytes = [], 0
    for ws in cell.ws:
        cnt = ws[off[1]:off[1] + 4 * E].cpu().numpy().view(np.int32)
        e = np.nonzero(cnt > 0)[0].astype(np.int32)
        ids.append(torch.from_numpy(e).cuda())
        nbytes += len(e) * cell.cfg.expert_bytes
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def timed(parts):
        def rnd():
            for l in range(cell.layers):
                xp.xp_stream_weights(cell.d, cell.model.tables[l], ids[l], sink, parts)
        rnd()
        torch.cuda.synchronize()
        g = _graph(rnd)
        g.replay()
        torch.cuda.synchronize()
        us = _replay_ms(g, 5) * 1e3 / cell.layers
        del g
        return us

    us = timed(7)
    per_layer = nbytes / cell.layers
    # the same bytes split as the two launches stream them: gate + up, then down
    gu_us, dn_us = timed(3), timed(4)
    return dict(us_per_layer=round(us, 3), gbps=round(per_layer / (us * 1e-6) / 1e9, 1),
                bytes_per_layer=int(per_layer), gateup_us=round(gu_us, 3), down_us=round(dn_us, 3),
                two_launch_us=round(gu_us + dn_us, 3))


PATHS = {"four_calls": ("route", "gateup", "down", "combine"), "two_calls": ("route_gateup", "down_combine"),
         "bf16_storage": ("route", "gateup_act16", "down_act16", "combine_y16"),
         "prefill": ("route", "prefill_gateup", "prefill_down", "combine")}
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PREFILL_LAYERS = 4               # prefill cells rotate over this many layers (3.4 GB of weights each)
# Pass-size sets timed against the default ({2,4,6,8} gate/up, {2,4} down):
# the padded passes of four the pages replaced, one size only, and powers of two.
TIER_SWEEP = [((4,), (4,)), ((8,), (4,)), ((2, 4, 8), (2, 4)), ((2,), (2,)), ((2, 4, 6, 8), (2, 4, 8))]
SWEEP_CELLS = ("four_same", "sixteen_random")


def _graph(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _replay_ms(g, reps: int) -> float:
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_cell(cell: Cell, path: str, steps: int, warmup: int) -> dict:
    """Round time of one path (graph of the 40-layer round), then each call's
    average duration: a graph of that call for every layer, back to back, timed
    with events on the launch stream (the plans are in place from the rounds)."""
    import torch
    kinds = PATHS[path]
    torch.cuda.synchronize()
    cell.round(kinds)                 # one eager round: plans in place, lazy init done
    torch.cuda.synchronize()
    g = _graph(lambda: cell.round(kinds))
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[steps]) / steps
    each = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    per = {}
    for kind in kinds:
        gk = _graph(lambda: [cell.call(kind, l) for l in range(cell.layers)])
        gk.replay()
        torch.cuda.synchronize()
        per[kind] = _replay_ms(gk, 5) * 1e3 / cell.layers
        del gk
    del g
    return dict(path=path, ms_per_round=ms, ms_min=each[0], ms_median=each[len(each) // 2], wall_s=wall,
                kernel_us=per)


def cell_report(cell: Cell, t: dict, copy_gbps: float, ceiling: dict | None = None) -> dict:
    cfg = cell.cfg
    st = cell.plan_stats()
    L = cell.layers
    H, I, k, R, E = cfg.H, cfg.I, cfg.k, cfg.R, cfg.E
    gu_w = 2 * (I * H // 2 + I * H // 32)            # gate+up bytes of one expert
    dn_w = H * I // 2 + H * I // 32
    distinct = sum(st["distinct"]) / L
    unique_bytes = distinct * cfg.expert_bytes
    layer_us = t["ms_per_round"] * 1e3 / L
    gbps = unique_bytes / (layer_us * 1e-6) / 1e9
    fused = t["path"] == "two_calls"
    b16 = t["path"] == "bf16_storage"
    gu_kind, dn_kind = ("route_gateup", "down_combine") if fused else (
        ("gateup_act16", "down_act16") if b16 else ("gateup", "down"))
    # algorithmic bytes of the gate/up launch: its distinct experts' gate+up weights, x read,
    # act written (+ logits read, top-k and plan written when it routes)
    act_b = 2 if b16 else 4
    gu_bytes = distinct * gu_w + R * H * 2 + R * k * I * act_b + ((R * E * 4 + R * k * 8) if fused else 0)
    # down: its experts' weights, act read, out written; the fused call also writes y, and
    # reads out back only when it runs as two launches (more than 64 (row, slot) entries)
    dn_bytes = distinct * dn_w + R * k * I * act_b + R * k * H * 4
    if fused:
        dn_bytes += R * H * 4 + (R * k * H * 4 if R * k > 64 else 0)
    gu_us, dn_us = t["kernel_us"][gu_kind], t["kernel_us"][dn_kind]
    # VALU lane-ops: one fma per weight per computed row (padding included), one
    # decode per two weights per pass, one scaled fma per group per row
    gu_rows = sum(st["gu_rows"]) / L
    dn_rows = sum(st["dn_rows"]) / L
    ops = gu_rows * 2 * I * H * (1 + 1 / 32) + dn_rows * H * I * (1 + 1 / 32)
    ops += (distinct * (2 * I * H + H * I)) / 2     # at least one decode pass per expert
    valu_us = ops / (CUS * LANES * CLOCK_GHZ * 1e9) * 1e6
    # weight bytes streamed again by an expert's second and later passes
    pass_bytes = (sum(st["gu_passes"]) * gu_w + sum(st["dn_passes"]) * dn_w) / L - distinct * (gu_w + dn_w)
    return dict(
        workload=cfg.name, path=t["path"], rows=R, layers=L,
        round_ms=round(t["ms_per_round"], 4), round_ms_fastest=round(t["ms_min"], 4),
        round_ms_median=round(t["ms_median"], 4), layer_us=round(layer_us, 3),
        rows_per_s=round(R / (t["ms_per_round"] / 1e3), 2),
        row_layers_per_s=round(R * L / (t["ms_per_round"] / 1e3), 1),
        distinct_experts=round(distinct, 2), unique_weight_bytes=int(unique_bytes),
        weight_gbps=round(gbps, 1), pct_hbm_peak=round(100 * gbps / HBM_PEAK_GBPS, 2),
        pct_copy_bw=round(100 * gbps / copy_gbps, 2),
        kernel_us={kk: round(v, 3) for kk, v in t["kernel_us"].items()},
        gateup_kernel=gu_kind, gateup_gbps=round(gu_bytes / (gu_us * 1e-6) / 1e9, 1), gateup_bytes=int(gu_bytes),
        down_kernel=dn_kind, down_gbps=round(dn_bytes / (dn_us * 1e-6) / 1e9, 1), down_bytes=int(dn_bytes),
        valu_bound_us=round(valu_us, 2), pass_bytes=int(round(pass_bytes)),
    ) | ({} if ceiling is None else dict(
        stream_ceiling_us=ceiling["us_per_layer"], stream_ceiling_gbps=ceiling["gbps"],
        pct_stream_ceiling=round(100 * ceiling["us_per_layer"] / layer_us, 2),
        stream_ceiling_two_launch_us=ceiling["two_launch_us"],
        pct_two_launch_ceiling=round(100 * ceiling["two_launch_us"] / layer_us, 2)))


def prefill_report(cell: Cell, t: dict) -> dict:
    """The prompt chunk on the matrix-core path: algorithmic flops are 6*H*I per
    (row, slot) pair (gate and up 2*H*I each, down 2*H*I); the down contraction
    runs twice (act as bf16 hi and lo), which the flop count does not include."""
    cfg = cell.cfg
    st = cell.plan_stats()
    L = cell.layers
    H, I, k, R = cfg.H, cfg.I, cfg.k, cfg.R
    pairs = R * k
    layer_ms = t["ms_per_round"] / L
    flops = 6.0 * H * I * pairs
    gu_us, dn_us = t["kernel_us"]["prefill_gateup"], t["kernel_us"]["prefill_down"]
    gu_tf = 4.0 * H * I * pairs / (gu_us * 1e-6) / 1e12
    dn_tf = 2.0 * H * I * pairs / (dn_us * 1e-6) / 1e12
    tf = flops / (layer_ms * 1e-3) / 1e12
    return dict(
        workload=cfg.name, path=t["path"], rows=R, layers=L, round_ms=round(t["ms_per_round"], 4),
        layer_ms=round(layer_ms, 4), rows_per_s=round(R / (layer_ms * 1e-3), 1),
        distinct_experts=round(sum(st["distinct"]) / L, 2),
        tflop_per_layer=round(flops / 1e12, 4), tflops=round(tf, 1),
        pct_mfma_peak=round(100 * tf / MFMA_BF16_PEAK_TFLOPS, 2),
        kernel_us={kk: round(v, 2) for kk, v in t["kernel_us"].items()},
        gateup_tflops=round(gu_tf, 1), down_tflops=round(dn_tf, 1),
        weight_gbps=round(sum(st["distinct"]) / L * cfg.expert_bytes / (layer_ms * 1e-3) / 1e9, 1),
    )


# ------------------------------------------------- dense FP8 projections
# A decode layer's dense FP8 projections at the layer's hidden width (synthetic
# shapes, N x K): a narrow one with a ragged last 128-column block, a medium, a
# square and one with K = 2048. E4M3FN weights, one fp32 scale per 128 x 128.
FP8_SHAPES = ((576, 4096), (1536, 4096), (4096, 4096), (4096, 2048))
FP8_ROWS = (1, 8, 16)
FP8_SEEDED_SETS = 4     # distinct seeded weight sets; the 40 layers hold copies in their own buffers


class Fp8Cell:
    """40 layers of the FP8 projection set, each in its own device buffers."""

    def __init__(self, layers: int):
        import numpy as np
        import torch
        import synth
        from fp4_routed_expert_xp_amd import xp
        self.layers = layers
        seeded = []
        for l in range(min(layers, FP8_SEEDED_SETS)):
            mats = []
            for i, (N, K) in enumerate(FP8_SHAPES):
                w = torch.from_numpy(synth.fp8_weights(5001, 16 * l + i, N, K)).cuda()
                packed = torch.empty(N * K, dtype=torch.uint8, device="cuda")
                xp.xp_fp8_pack(w, packed)
                sc = torch.from_numpy(synth.fp8_scales(5001, 16 * l + i, N, K)).cuda()
                mats.append((packed, sc))
            seeded.append(mats)
        self.mats = [[(p.clone(), sc.clone()) for p, sc in seeded[l % len(seeded)]] for l in range(layers)]
        del seeded
        rmax = max(FP8_ROWS)
        kmax = max(K for _, K in FP8_SHAPES)
        nmax = max(N for N, _ in FP8_SHAPES)
        xb = synth.activations(5002, 0, rmax, kmax)
        self.x = torch.from_numpy(xb.view(np.int16).copy()).cuda()
        self.xf = torch.from_numpy(synth.bf16_bits_to_f32(xb) + np.float32(1.0 / 3.0)).cuda()  # full fp32 values
        self.y = torch.empty((rmax, nmax), dtype=torch.float32, device="cuda")
        self.ys = [torch.empty((rmax, N), dtype=torch.float32, device="cuda") for N, _ in FP8_SHAPES]
        self.set_bytes = sum(N * K + ((N + 127) // 128) * (K // 128) * 4 for N, K in FP8_SHAPES)
        torch.cuda.synchronize()


def time_fp8(cell: Fp8Cell, steps: int, warmup: int) -> dict:
    """Per row count: the round (every projection of every layer, one graph) and
    each shape alone (a graph of that shape over the layers)."""
    import torch
    out = {}
    for R in FP8_ROWS:
        xs = {K: cell.x[:R, :K].contiguous() for _, K in FP8_SHAPES}

        def run(i, l):
            from fp4_routed_expert_xp_amd import xp
            N, K = FP8_SHAPES[i]
            packed, sc = cell.mats[l][i]
            xp.xp_fp8_rows(R, N, K, xs[K], packed, sc, cell.y, 0)

        def rnd():
            for l in range(cell.layers):
                for i in range(len(FP8_SHAPES)):
                    run(i, l)
        rnd()
        torch.cuda.synchronize()
        g = _graph(rnd)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        ms = _replay_ms(g, steps)
        del g
        # the same round with one launch per layer for the projections that share x (same K)
        by_k = {}
        for i, (N, K) in enumerate(FP8_SHAPES):
            by_k.setdefault(K, []).append(i)

        def rnd_multi():
            from fp4_routed_expert_xp_amd import xp
            for l in range(cell.layers):
                for K, idx in by_k.items():
                    mats = [(cell.mats[l][i][0], cell.mats[l][i][1], cell.ys[i]) for i in idx]
                    xp.xp_fp8_rows_multi(R, K, xs[K], mats)
        rnd_multi()
        torch.cuda.synchronize()
        g = _graph(rnd_multi)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        ms_multi = _replay_ms(g, steps)
        del g
        xfs = {K: cell.xf[:R, :K].contiguous() for _, K in FP8_SHAPES}

        def run_f32(i, l):
            from fp4_routed_expert_xp_amd import xp
            N, K = FP8_SHAPES[i]
            packed, sc = cell.mats[l][i]
            xp.xp_fp8_rows_f32(R, N, K, xfs[K], packed, sc, cell.y, 0)

        per, per_f32 = {}, {}
        for i, (N, K) in enumerate(FP8_SHAPES):
            for fn, dst in ((run, per), (run_f32, per_f32)):
                gk = _graph(lambda: [fn(i, l) for l in range(cell.layers)])
                gk.replay()
                torch.cuda.synchronize()
                dst["%dx%d" % (N, K)] = round(_replay_ms(gk, 5) * 1e3 / cell.layers, 3)
                del gk
        layer_us = ms * 1e3 / cell.layers
        multi_us = ms_multi * 1e3 / cell.layers
        out[R] = dict(rows=R, round_ms=round(ms, 4), layer_us=round(layer_us, 3),
                      weight_gbps=round(cell.set_bytes / (layer_us * 1e-6) / 1e9, 1),
                      pct_hbm_peak=round(100 * cell.set_bytes / (layer_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
                      multi=dict(launches_per_layer=len(by_k), round_ms=round(ms_multi, 4),
                                 layer_us=round(multi_us, 3),
                                 weight_gbps=round(cell.set_bytes / (multi_us * 1e-6) / 1e9, 1),
                                 pct_hbm_peak=round(100 * cell.set_bytes / (multi_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                                                    2)),
                      kernel_us=per, kernel_us_f32_rows=per_f32)
    return out


# ------------------------------------------------------------ CPU baseline
def cpu_baseline(budget_s: float) -> dict:
    """The float64 oracle, untuned, on this host's cores: one-row layers of the
    release-width synthetic model until about budget_s of CPU time is spent."""
    import numpy as np
    import oracle
    import synth
    cfg = synth.CONFIGS["one_row"]
    times, threads = [], 1
    cpu0 = time.process_time()
    l = 0
    while True:
        x, lg = synth.layer_inputs(cfg, l, plant=False)
        ids, _ = oracle.route(lg, cfg.k)
        ex = {int(e): synth.layer_expert(cfg, l, int(e)) for e in np.unique(ids)}
        c0 = time.process_time()
        t0 = time.perf_counter()
        res = oracle.layer(x, lg, ex, cfg.H, cfg.I, cfg.E, cfg.k)
        times.append(time.perf_counter() - t0)
        threads = min(res["threads"], cfg.R * cfg.k)
        l += 1
        if time.process_time() - cpu0 >= budget_s or l >= 8 or (time.process_time() - c0) * (l + 1) > 4 * budget_s:
            break
    per_layer = sum(times) / len(times)
    # the multi-row workloads, one layer each, for context (same oracle, same threads)
    others = {}
    for name in ("four_same", "sixteen_random"):
        c2 = synth.CONFIGS[name]
        x, lg = synth.layer_inputs(c2, 0, plant=False)
        ids, _ = oracle.route(lg, c2.k)
        ex = {int(e): synth.layer_expert(c2, 0, int(e)) for e in np.unique(ids)}
        t0 = time.perf_counter()
        oracle.layer(x, lg, ex, c2.H, c2.I, c2.E, c2.k)
        dt = time.perf_counter() - t0
        others[name] = dict(rows_per_s=round(c2.R / (dt * 40), 4), s_per_layer=round(dt, 3))
    # one layer of the one-row round on a single thread, for the per-core figure
    omp_default = oracle.omp_threads()
    x, lg = synth.layer_inputs(cfg, 0, plant=False)
    ids, _ = oracle.route(lg, cfg.k)
    ex = {int(e): synth.layer_expert(cfg, 0, int(e)) for e in np.unique(ids)}
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.layer(x, lg, ex, cfg.H, cfg.I, cfg.E, cfg.k)
        single = time.perf_counter() - t0
    finally:
        oracle.set_threads(omp_default)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return dict(value=round(cfg.R / (per_layer * 40), 4), unit="rows/s", cores=int(threads), kind="oracle",
                sample="%d of the 40 layers of the one-row round (1 row x 8 experts each), float64 C oracle, "
                       "OpenMP over (row, slot) pairs; %.3f s per layer, scaled to a 40-layer round" %
                       (len(times), per_layer),
                host={"cpu": model, "logical_cpus": os.cpu_count()}, other_workloads=others,
                single_thread=dict(value=round(cfg.R / (single * 40), 4), unit="rows/s", cores=1,
                                   s_per_layer=round(single, 3),
                                   sample="layer 0 of the one-row round on one thread, scaled to 40 layers"))


DECODE_CELLS = ("one_row", "four_same", "sixteen_random")


def decode_pct(reports: dict) -> dict:
    """% of the HBM peak on expert-weight bytes of the two-call path per decode
    workload (1, 4 and 16 rows), their minimum, and the same against the
    read-only stream ceiling."""
    out = {}
    for name in DECODE_CELLS:
        r = reports.get("%s/two_calls" % name)
        if r is not None:
            out["%d_rows" % r["rows"]] = r["pct_hbm_peak"]
            if "pct_stream_ceiling" in r:
                out["%d_rows_vs_stream_ceiling" % r["rows"]] = r["pct_stream_ceiling"]
    peaks = [v for kk, v in out.items() if kk.endswith("_rows")]
    if peaks:
        out["min"] = min(peaks)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    from fp4_routed_expert_xp_amd import xp
    xp.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cells = [c for c in args.cells.split(",") if c]
    base = synth.CONFIGS["one_row"]
    t0 = time.perf_counter()
    log("materialising %d layers x %d experts (%.1f GB)" % (args.layers, base.E,
                                                             args.layers * base.E * base.expert_bytes / 1e9))
    model = Model(base, args.layers)
    log("weights ready in %.1f s" % (time.perf_counter() - t0))
    copy_gbps = copy_bandwidth_gbps()
    log("plain copy bandwidth %.0f GB/s" % copy_gbps)
    reports, timings = {}, {}
    for name in cells:
        if name == "fp8_rows":
            fcell = Fp8Cell(args.layers)
            for R, rep in time_fp8(fcell, args.steps, args.warmup).items():
                rep["bytes_per_layer"] = fcell.set_bytes
                rep["shapes"] = ["%dx%d" % s for s in FP8_SHAPES]
                reports["fp8_rows/%d" % R] = rep
                log("fp8_rows/%d: %s" % (R, json.dumps(rep)))
            del fcell
            continue
        cfg = synth.CONFIGS[name]
        if name == "prefill":
            cell = Cell(model, cfg, min(args.layers, PREFILL_LAYERS))
            t = time_cell(cell, "prefill", args.steps, args.warmup)
            key = "prefill/prefill"
            timings[key] = t
            reports[key] = prefill_report(cell, t)
            log("%s: %s" % (key, json.dumps(reports[key])))
            del cell
            continue
        cell = Cell(model, cfg, args.layers)
        ceiling = None
        for path in ("two_calls", "four_calls", "bf16_storage"):
            t = time_cell(cell, path, args.steps, args.warmup)
            if ceiling is None:     # the plans are in place after the first path's rounds
                ceiling = time_stream(cell)
                log("%s: read-only stream ceiling %s" % (name, json.dumps(ceiling)))
            key = "%s/%s" % (name, path)
            timings[key] = t
            reports[key] = cell_report(cell, t, copy_gbps, ceiling)
            log("%s: %s" % (key, json.dumps(reports[key])))
        if name in SWEEP_CELLS and not args.no_tier_sweep:
            # same rows, other pass sizes: the bits are unchanged (the probe
            # tests check it), only the time moves
            in_force = xp.xp_get_tiers()
            for gu, dn in TIER_SWEEP:
                xp.xp_set_tiers(list(gu), list(dn))
                try:
                    t = time_cell(cell, "two_calls", args.steps, args.warmup)
                finally:
                    xp.xp_set_tiers(*in_force)
                key = "%s/two_calls/tiers_gu%s_dn%s" % (name, "-".join(map(str, gu)), "-".join(map(str, dn)))
                rep = cell_report(cell, t, copy_gbps, ceiling)
                rep["tiers"] = {"gate_up": list(gu), "down": list(dn)}
                reports[key] = rep
                log("%s: %s" % (key, json.dumps(rep)))
    decode = [c for c in cells if c not in ("prefill", "fp8_rows")]
    if not decode:
        log("the headline is a decode workload: name one of one_row, four_same, sixteen_random in --cells")
        sys.exit(2)
    head_key = "%s/two_calls" % decode[0]
    head = reports[head_key]
    th = timings[head_key]
    achieved = head["gateup_gbps"]
    line = {
        "metric": METRIC,
        "value": head["rows_per_s"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["round_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded fp4 e2m1 codes, E4M3 2^U{-6..0} scales, bf16 N(0,1) x, N(0,1) logits)",
        "config": {"workload": "%s: %d-row decode through a %d-layer round of independent layers, hidden %d, "
                               "intermediate %d, %d experts, top-%d; two launches per layer "
                               "(xp_route_gateup, xp_down_combine)" % (decode[0], head["rows"], args.layers,
                                                                        base.H, base.I, base.E, base.k),
                   "rows": head["rows"], "layers": args.layers, "hidden": base.H, "inter": base.I,
                   "experts": base.E, "top_k": base.k, "path": "two_calls",
                   "pass_sizes": dict(zip(("gate_up", "down"), xp.xp_get_tiers()))},
        "roofline": {"kernel": "gateup_one_row_kernel (xp_route_gateup)" if head["rows"] == 1
                     else "route_*_kernel + gateup_kernel<0> (xp_route_gateup)", "bound": "hbm",
                     "achieved": round(achieved, 1), "bytes_per_launch": head["gateup_bytes"],
                     "launch_us": head["kernel_us"]["route_gateup"],
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic()},
        "copy_gbps": round(copy_gbps, 1),
        "decode_pct_hbm_peak": decode_pct(reports),
        "wall_s_timed": round(th["wall_s"], 4),
        "cells": reports,
    }
    dn_kernel = "down_combine_one_row_kernel (xp_down_combine)" if head["rows"] == 1 else (
        "down_combine_rows_kernel (xp_down_combine)" if head["rows"] * base.k <= 64
        else "down_kernel<false> + combine_kernel<false> (xp_down_combine)")
    line["roofline_down"] = {
        "kernel": dn_kernel, "bound": "hbm", "achieved": head["down_gbps"], "bytes_per_launch": head["down_bytes"],
        "launch_us": head["kernel_us"]["down_combine"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(head["down_gbps"] / HBM_PEAK_GBPS, 4),
        "traffic": measured_traffic(DOWN_TRAFFIC) if head["rows"] == 1 else None}
    if "prefill/prefill" in reports:
        pf = reports["prefill/prefill"]
        cfg = synth.CONFIGS["prefill"]
        line["prefill_roofline"] = {
            "kernel": "prefill_gateup_kernel (xp_prefill_gateup)", "bound": "mfma",
            "achieved": pf["gateup_tflops"], "flops_per_launch": 4 * cfg.H * cfg.I * cfg.R * cfg.k,
            "launch_us": pf["kernel_us"]["prefill_gateup"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(pf["gateup_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(PF_GU_TRAFFIC, PREFILL_SOURCES)}
        line["prefill_roofline_down"] = {
            "kernel": "prefill_down_kernel (xp_prefill_down)", "bound": "mfma",
            "achieved": pf["down_tflops"], "flops_per_launch": 2 * cfg.H * cfg.I * cfg.R * cfg.k,
            "launch_us": pf["kernel_us"]["prefill_down"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(pf["down_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(PF_DN_TRAFFIC, PREFILL_SOURCES)}
    fp8 = [reports[k] for k in ("fp8_rows/1", "fp8_rows/16") if k in reports]
    if fp8:
        N, K = 4096, 4096
        us = fp8[0]["kernel_us"]["%dx%d" % (N, K)]
        nbytes = N * K + (N // 128) * (K // 128) * 4 + 2 * K + 4 * N
        line["fp8_roofline"] = {
            "kernel": "fp8_rows_kernel (xp_fp8_rows, %dx%d, %d row)" % (N, K, fp8[0]["rows"]), "bound": "hbm",
            "achieved": round(nbytes / (us * 1e-6) / 1e9, 1), "bytes_per_launch": nbytes, "launch_us": us,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(FP8_TRAFFIC, FP8_SOURCES)}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
