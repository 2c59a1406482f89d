"""GPU: the prefill-chunk contraction (xp_prefill_gateup, xp_prefill_down) against the oracle.

The matrix-core path sums in another order than the decode chain, so it is held
to the per-row tolerance against the float64 oracle (max |gpu - ref| / max |ref|
<= 1e-3 over each row's entries of act, out and y) and not to bit equality.
Small widths cover several 128-row blocks per expert with ragged tails, a
column count that leaves half of the last 128-column block empty, and single
rows; the 4,096-row chunk at release widths is checked on sampled rows (routing
and the plan for every row) since the oracle cannot finish the whole chunk in
seconds.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from fp4_routed_expert_xp_amd import xp

from gpu_helpers import DeviceLayer, log, read_plan, rel_err_rows, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3
TINY = synth.CONFIGS["tiny"]
# 384 intermediate columns: three 128-column blocks for gate/up, the last one half empty.
MID = dataclasses.replace(TINY, name="mid", H=512, I=384, E=16, k=4, seed=1101, weight_seed=1101)
PREFILL = synth.CONFIGS["prefill"]
# Widths that are multiples of 64 only: gate/up's second 128-column item has one
# live 64-column tile, down's second 256-column item one live tile of four, and
# the group counts (10 and 6) take the shallow weight ring.
ODD = dataclasses.replace(TINY, name="odd", H=320, I=192, E=8, k=3, seed=1111, weight_seed=1111)


def run_prefill(layer: DeviceLayer, x_bits, logits) -> dict:
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
    xp.xp_route_bucket(d, R, lg, topk_id, topk_w, ws)
    xp.xp_prefill_gateup(d, R, x, layer.table, ws, act)
    xp.xp_prefill_down(d, R, act, layer.table, ws, out)
    xp.xp_combine(d, R, out, topk_w, y)
    torch.cuda.synchronize()
    return dict(topk_id=topk_id.cpu().numpy(), topk_w=topk_w.cpu().numpy(), act=act.cpu().numpy(),
                out=out.cpu().numpy(), y=y.cpu().numpy(), ws=ws.cpu().numpy())


def oracle_rows(layer: DeviceLayer, x, lg):
    ids, _ = oracle.route(lg, layer.cfg.k)
    ex = {int(e): layer.host_expert(int(e)) for e in np.unique(ids)}
    return oracle.layer(x, lg, ex, layer.cfg.H, layer.cfg.I, layer.cfg.E, layer.cfg.k)


def check_rows(res, ref, rows=None):
    sel = slice(None) if rows is None else rows
    assert np.array_equal(res["topk_id"][sel], ref["topk_id"])
    for name in ("act", "out", "y"):
        got = res[name][sel]
        assert np.all(np.isfinite(got)), name
        err = rel_err_rows(got, ref[name])
        assert np.all(err <= TOL), (name, float(err.max()), int(err.argmax()))
    return max(float(rel_err_rows(res[n][sel], ref[n]).max()) for n in ("act", "out", "y"))


@pytest.fixture(scope="module")
def tiny_layer():
    return DeviceLayer(TINY, 0)


@pytest.fixture(scope="module")
def mid_layer():
    return DeviceLayer(MID, 0)


@pytest.mark.parametrize("R", [1, 3, 64, 300, 1000])
def test_tiny_prefill_matches_oracle(tiny_layer, R):
    # 8 experts, top-2: R = 1000 puts about 250 rows on each expert (two full
    # 128-row blocks and a ragged third).
    log("prefill tiny R=%d" % R)
    x = synth.activations(TINY.seed, 100 + R, R, TINY.H)
    lg = synth.logits(TINY.seed, 100 + R, R, TINY.E)
    res = run_prefill(tiny_layer, x, lg)
    ref = oracle_rows(tiny_layer, x, lg)
    worst = check_rows(res, ref)
    log("  worst per-row relative error %.2e" % worst)


@pytest.mark.parametrize("R", [2, 129, 517])
def test_mid_prefill_matches_oracle(mid_layer, R):
    log("prefill mid R=%d" % R)
    x = synth.activations(MID.seed, R, R, MID.H)
    lg = synth.logits(MID.seed, R, R, MID.E, bias_sigma=0.5)
    res = run_prefill(mid_layer, x, lg)
    ref = oracle_rows(mid_layer, x, lg)
    worst = check_rows(res, ref)
    log("  worst per-row relative error %.2e" % worst)


@pytest.mark.parametrize("R", [5, 300])
def test_odd_widths_prefill_matches_oracle(R):
    layer = DeviceLayer(ODD, 0)
    log("prefill odd widths H=%d I=%d R=%d" % (ODD.H, ODD.I, R))
    x = synth.activations(ODD.seed, R, R, ODD.H)
    lg = synth.logits(ODD.seed, R, R, ODD.E, bias_sigma=0.5)
    res = run_prefill(layer, x, lg)
    ref = oracle_rows(layer, x, lg)
    worst = check_rows(res, ref)
    log("  worst per-row relative error %.2e" % worst)


def test_prefill_repeated_on_one_plan(tiny_layer):
    # Each call zeroes its work counters in the workspace header before its
    # contraction, so calls repeated on one plan give the same bits.
    R = 300
    d = tiny_layer.d
    x = to_dev(synth.activations(TINY.seed, 31, R, TINY.H))
    lg = to_dev(synth.logits(TINY.seed, 31, R, TINY.E).astype(np.float32))
    ws = torch.zeros(max(xp.xp_workspace_bytes(d, R), 256), dtype=torch.uint8, device="cuda")
    topk_id = torch.empty((R, d.top_k), dtype=torch.int32, device="cuda")
    topk_w = torch.empty((R, d.top_k), dtype=torch.float32, device="cuda")
    xp.xp_route_bucket(d, R, lg, topk_id, topk_w, ws)
    acts, outs = [], []
    for _ in range(3):
        act = torch.full((R, d.top_k, d.inter), float("nan"), dtype=torch.float32, device="cuda")
        out = torch.full((R, d.top_k, d.hidden), float("nan"), dtype=torch.float32, device="cuda")
        xp.xp_prefill_gateup(d, R, x, tiny_layer.table, ws, act)
        xp.xp_prefill_down(d, R, act, tiny_layer.table, ws, out)
        torch.cuda.synchronize()
        acts.append(act.cpu().numpy().view(np.uint32))
        outs.append(out.cpu().numpy().view(np.uint32))
    for i in (1, 2):
        assert np.array_equal(acts[i], acts[0]) and np.array_equal(outs[i], outs[0])
    assert np.all(np.isfinite(acts[0].view(np.float32))) and np.all(np.isfinite(outs[0].view(np.float32)))


def test_prefill_skewed_expert(tiny_layer):
    # Every row on experts 0 and 1 (one expert with all R rows in slot 0):
    # ten full blocks and a tail of 5.
    R = 1285
    log("prefill tiny skewed R=%d" % R)
    x = synth.activations(TINY.seed, 7, R, TINY.H)
    lg = np.full((R, TINY.E), -4.0, dtype=np.float32)
    lg[:, 0] = 3.0
    lg[:, 1] = 2.0 + 0.001 * np.arange(R, dtype=np.float32) / R
    res = run_prefill(tiny_layer, x, lg)
    ref = oracle_rows(tiny_layer, x, lg)
    check_rows(res, ref)


def test_prefill_empty_and_errors(tiny_layer):
    d = tiny_layer.d
    xp.xp_prefill_gateup(d, 0, None, tiny_layer.table, None, None)
    xp.xp_prefill_down(d, 0, None, tiny_layer.table, None, None)
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    x = torch.zeros((4, d.hidden), dtype=torch.int16, device="cuda")
    act = torch.zeros((4, d.top_k, d.inter), dtype=torch.float32, device="cuda")
    with pytest.raises(xp.XPError) as ei:
        xp.xp_prefill_gateup(d, 4, x, tiny_layer.table, ws, act)
    assert ei.value.status == xp.XP_ERR_WORKSPACE


@pytest.fixture(scope="module")
def prefill_layer():
    log("materialising release-width layer 0 (256 experts) for the prefill chunk")
    return DeviceLayer(PREFILL, 0)


def slab_class(rows_in_block: int) -> int:
    """16-row slabs a 128-row block of an expert computes: its rows rounded up to a multiple of 16."""
    return (rows_in_block + 15) // 16


def merged_first_row(n: int):
    """Gate/up computes an expert of n rows whose last 128-row block has at most
    32 rows after a full one as one item of n - 128 (b - 1) rows, b its block
    count (9 or 10 slabs); returns that item's first row within the expert, or
    None when the expert has no such item."""
    b = (n + 127) // 128
    return 128 * (b - 2) if b >= 2 and n - 128 * (b - 1) <= 32 else None


def shape_chosen_rows(count, offset, entry, k, R, seed=5):
    """Rows of a chunk picked by the work items they fall in: for every slab count
    1 to 8, the first and last row of the last (ragged) block of two experts of
    that class; for gate/up's merged items of 9 and 10 slabs, the first row of
    two such items of each count; the last row of the busiest expert's ragged block and the first
    row of one of its full blocks; every row of the least-loaded routed expert
    (up to four); the first and last chunk rows; and random rows up to 40."""
    rows = set([0, R - 1])
    E = len(count)
    routed = [e for e in range(E) if count[e] > 0]
    members = lambda e: [int(entry[i]) // k for i in range(offset[e], offset[e + 1])]
    by_class = {c: [] for c in range(1, 11)}
    for e in routed:
        last = count[e] - 128 * ((count[e] - 1) // 128)
        by_class[slab_class(last)].append(e)
        if merged_first_row(count[e]) is not None:
            by_class[slab_class(count[e] - merged_first_row(count[e]))].append(e)
    for cls, es in by_class.items():
        for e in es[:2]:
            m = members(e)
            b0 = 128 * ((len(m) - 1) // 128)
            rows.update([m[b0], m[-1]])
            if cls > 8:
                rows.add(m[merged_first_row(len(m))])
    busiest = int(np.argmax(count))
    m = members(busiest)
    rows.add(m[-1])
    if len(m) > 128:
        rows.add(m[128 * ((len(m) - 1) // 128) - 128])   # first row of its last full block
    least = min(routed, key=lambda e: count[e])
    rows.update(members(least)[:4])
    rng = np.random.default_rng(seed)
    while len(rows) < 40:
        rows.add(int(rng.integers(0, R)))
    return sorted(rows), by_class, busiest, least


def test_prefill_chunk_release_width(prefill_layer):
    """4,096 rows, 256 experts, top-8, logits with a per-expert bias (sigma 0.5).

    Routing, counts, offsets and entries are bit-exact for every row; act, out
    and y are compared with the float64 oracle on 40 rows chosen by the work
    item they fall in (every slab count of an expert's ragged last block, the
    busiest expert's full and ragged blocks, the least-loaded expert) plus
    random rows; the whole chunk is checked to be finite. Gate/up's merged
    items (a full block with a last block of at most 32 rows, 9 or 10 slabs) are
    among the slab counts.
    """
    cfg = PREFILL
    x, lg = synth.layer_inputs(cfg, 0)
    log("prefill chunk: R=%d" % cfg.R)
    res = run_prefill(prefill_layer, x, lg)
    ids, w = oracle.route(lg, cfg.k)
    assert np.array_equal(res["topk_id"], ids)
    count, offset, entry = oracle.bucket(ids, cfg.E)
    plan = read_plan(prefill_layer.d, cfg.R, res["ws"])
    assert np.array_equal(plan["count"], count)
    assert np.array_equal(plan["offset"], offset)
    assert np.array_equal(plan["entry"], entry)
    for name in ("act", "out", "y"):
        assert np.all(np.isfinite(res[name])), name
    rows, by_class, busiest, least = shape_chosen_rows(count, offset, entry, cfg.k, cfg.R)
    log("  busiest expert %d with %d rows, least-loaded %d with %d; %d experts routed; experts per slab count %s"
        % (busiest, count[busiest], least, count[least], int((count > 0).sum()),
           {c: len(v) for c, v in by_class.items()}))
    assert all(len(v) > 0 for v in by_class.values()), "the chunk exercises every slab count"
    assert len(rows) >= 32
    ref = oracle_rows(prefill_layer, x[rows], lg[rows])
    worst = check_rows(res, ref, rows)
    log("  %d chosen rows: worst per-row relative error %.2e" % (len(rows), worst))


# hidden 1536: an odd number (three) of 512-column down items per row block
WIDE = dataclasses.replace(TINY, name="wide", H=1536, I=256, E=16, k=4, seed=1121, weight_seed=1121)


@pytest.mark.parametrize("R", [5, 100, 600])
def test_short_last_blocks_match_oracle(R):
    """Experts whose last row block has at most two slabs, against the float64
    oracle on every row: few rows per expert (every block short), and 150 rows
    per expert on average (full blocks and short ones side by side, which
    gate/up computes as single items of 129 to 160 rows)."""
    layer = DeviceLayer(WIDE, 0)
    x = synth.activations(WIDE.seed, R, R, WIDE.H)
    lg = synth.logits(WIDE.seed, R, R, WIDE.E, bias_sigma=0.5)
    res = run_prefill(layer, x, lg)
    count = np.bincount(res["topk_id"].ravel(), minlength=WIDE.E)
    tails = int(np.sum((count > 0) & (count - ((count - 1) // 128) * 128 <= 32)))
    merged = sum(merged_first_row(int(n)) is not None for n in count)
    log("wide R=%d: %d experts with a last block of at most 32 rows, %d after a full block" % (R, tails, merged))
    assert tails > 0
    if R == 600:
        assert merged > 0
    worst = check_rows(res, oracle_rows(layer, x, lg))
    log("  worst per-row relative error %.2e" % worst)


# Expert row counts on both sides of gate/up's merge rule (a last 128-row block
# of at most 32 rows joins the full block before it): 129..160 and 288 merge,
# 161 and 289 do not; 128 is one full block, 32 and 33 a lone short block.
BOUNDARY_COUNTS = [129, 144, 145, 160, 161, 288, 289, 32, 33, 1, 128, 17, 0, 16, 57, 68]


def routed_logits(counts, R, k, seed):
    """Logits that route exactly counts[e] of the R rows' k slots to expert e:
    the experts' slots laid out expert by expert and written column-major into
    an R x k table (every count at most R, so no row gets an expert twice);
    row r gives its k experts logits k, k-1, .., 1 in column order and every
    other expert a value in [-2, -1)."""
    E = len(counts)
    assert sum(counts) == R * k and max(counts) <= R
    seq = np.repeat(np.arange(E), counts)
    table = seq.reshape(k, R).T
    rng = np.random.default_rng(seed)
    lg = (-2.0 + rng.random((R, E))).astype(np.float32)
    for j in range(k):
        lg[np.arange(R), table[:, j]] = np.float32(k - j)
    return lg


def test_merge_boundaries_match_oracle():
    """Experts with exactly 129, 144, 145, 160 (one gate/up item of 9 or 10
    slabs), 161 (a full item and a three-slab one), 288 (two items, the second
    of 160 rows) and 289 rows, beside experts of 0, 1, 16, 17, 32, 33, 57, 68
    and 128 rows, against the float64 oracle on every row."""
    R = sum(BOUNDARY_COUNTS) // WIDE.k
    layer = DeviceLayer(WIDE, 0)
    x = synth.activations(WIDE.seed, R, R, WIDE.H)
    lg = routed_logits(BOUNDARY_COUNTS, R, WIDE.k, seed=77)
    res = run_prefill(layer, x, lg)
    plan = read_plan(layer.d, R, res["ws"])
    assert np.array_equal(plan["count"], np.array(BOUNDARY_COUNTS))
    worst = check_rows(res, oracle_rows(layer, x, lg))
    log("merge boundaries R=%d: worst per-row relative error %.2e" % (R, worst))


def test_prefill_largest_experts_and_topk():
    """1024 experts and top-16 (four experts per thread in the workgroups' block scan)."""
    cfg = dataclasses.replace(TINY, name="maxed", H=128, I=64, E=1024, k=16, seed=1202, weight_seed=1202)
    layer = DeviceLayer(cfg, 0)
    R = 300
    x = synth.activations(cfg.seed, R, R, cfg.H)
    lg = synth.logits(cfg.seed, R, R, cfg.E, bias_sigma=0.5)
    res = run_prefill(layer, x, lg)
    check_rows(res, oracle_rows(layer, x, lg))


@pytest.mark.parametrize("pieces", [(1, 7, 100, 300), (64, 64, 64, 64, 64)])
def test_prefill_rows_do_not_depend_on_the_chunk(mid_layer, pieces):
    """A row's act, out and y bits are the same whether it runs in a 700-row
    chunk or in a piece of 1, 7, 64, 100 or 300 rows: each output element is
    one row of A against one column of B, accumulated over K in a fixed group
    order, whatever else shares the 128-row block."""
    R = 700
    x = synth.activations(MID.seed + 3, R, R, MID.H)
    lg = synth.logits(MID.seed + 3, R, R, MID.E, bias_sigma=0.5)
    full = run_prefill(mid_layer, x, lg)
    r0 = 0
    for n in pieces:
        part = run_prefill(mid_layer, x[r0:r0 + n], lg[r0:r0 + n])
        for name in ("act", "out", "y"):
            a = np.ascontiguousarray(full[name][r0:r0 + n]).view(np.uint32)
            b = np.ascontiguousarray(part[name]).view(np.uint32)
            assert np.array_equal(a, b), (pieces, r0, n, name)
        r0 += n


def test_prefill_chunk_invariance_release_width(prefill_layer):
    """The same at release widths: rows of the 4,096-row chunk against pieces
    of 1, 7 and 100 rows cut from it (busiest-expert rows included)."""
    cfg = PREFILL
    x, lg = synth.layer_inputs(cfg, 0)
    full = run_prefill(prefill_layer, x, lg)
    for r0, n in ((0, 1), (1, 7), (3996, 100)):
        part = run_prefill(prefill_layer, x[r0:r0 + n], lg[r0:r0 + n])
        for name in ("act", "out", "y"):
            a = np.ascontiguousarray(full[name][r0:r0 + n]).view(np.uint32)
            b = np.ascontiguousarray(part[name]).view(np.uint32)
            assert np.array_equal(a, b), (r0, n, name)


def test_prefill_general_scales():
    """Scale bytes over every finite E4M3FN value (negative, zero, subnormal,
    non-power-of-two) in a third of the groups and in some rows of another third;
    the rest powers of two, so both weight decodes of the kernels run in one launch."""
    from gpu_helpers import HostLayer
    cfg = MID
    experts = {e: synth.expert_mixed(cfg.weight_seed, 0, e, cfg.H, cfg.I, cfg.emin, cfg.emax) for e in range(cfg.E)}
    layer = HostLayer(cfg, experts)
    for R in (3, 300):
        log("prefill mid, general scales, R=%d" % R)
        x = synth.activations(cfg.seed, 500 + R, R, cfg.H)
        lg = synth.logits(cfg.seed, 500 + R, R, cfg.E, bias_sigma=0.5)
        res = run_prefill(layer, x, lg)
        ref = oracle_rows(layer, x, lg)
        worst = check_rows(res, ref)
        log("  worst per-row relative error %.2e" % worst)


def test_prefill_weight_decodes_agree_bit_for_bit():
    """The power-of-two weight decode and the general one give the same bf16
    weights. Layer B differs from layer A only in one scale byte per 32 columns
    and group, made 1.375 (0x3B) where that column's 32 codes of the group are
    +0, so B's weights equal A's; every wave-group of A runs the power-of-two
    decode and every wave-group of B the general one, and the outputs must be
    bit-equal."""
    from gpu_helpers import HostLayer, bits
    cfg = MID
    a_ex, b_ex = {}, {}
    for e in range(cfg.E):
        ex = synth.expert(cfg.weight_seed, 0, e, cfg.H, cfg.I, cfg.emin, cfg.emax)
        bx = {k: v.copy() for k, v in ex.items()}
        for m in ("gate", "up", "down"):
            codes, scales = ex[m + "_codes"], ex[m + "_scales"]
            N, G = scales.shape
            for g in range(G):
                for blk in range(N // 32):
                    n = 32 * blk + g % 32
                    codes[n, 16 * g:16 * g + 16] = 0
            bx[m + "_codes"] = codes.copy()
            sb = scales.copy()
            for g in range(G):
                for blk in range(N // 32):
                    sb[32 * blk + g % 32, g] = 0x3B
            bx[m + "_scales"] = sb
        a_ex[e], b_ex[e] = ex, bx
    la, lb = HostLayer(cfg, a_ex), HostLayer(cfg, b_ex)
    R = 300
    log("prefill mid, two weight decodes, R=%d" % R)
    x = synth.activations(cfg.seed, 700, R, cfg.H)
    lg = synth.logits(cfg.seed, 700, R, cfg.E, bias_sigma=0.5)
    ra, rb = run_prefill(la, x, lg), run_prefill(lb, x, lg)
    for name in ("act", "out", "y"):
        assert np.array_equal(bits(ra[name]), bits(rb[name])), name
    check_rows(ra, oracle_rows(la, x, lg))
