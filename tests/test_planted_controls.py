"""Planted controls, on the CPU: the probe's checks must go red for each mistake they exist to catch.

The GPU probe holds every row of a launch bit-equal to that row launched alone, and the
plan test holds the plan equal to the oracle's. Here a CPU model of a gate/up launch runs
over the oracle's plan (passes of 2/4/6/8 rows, padding rows repeating the last real row,
each row's fp32 chain, eight leaves and tree), and each control plants one mistake in that
model, never in the GPU kernels:

- rows read their pass's first row,
- padding rows are written,
- multi-row passes add the eight leaves in another order,
- bucketing keeps an expert's rows in arrival order of a racing writer (unstable).

The unplanted model passes the same checks, so each red result comes from the mistake.
The tree-order control is caught bit for bit but not by the 1e-3 tolerance, which is why
the probe compares bits.
"""
import numpy as np
import pytest

import oracle
import synth

CFG = synth.CONFIGS["tiny"]
GU_TIERS = (2, 4, 6, 8)
TREE = (((0, 1), (2, 3)), ((4, 5), (6, 7)))
TREE_SWAPPED = (((0, 2), (1, 3)), ((4, 6), (5, 7)))


def f32(v):
    return np.float32(v)


def leaves(W, x, G):
    """Eight fp32 leaves per column: group g's 32 products (weights with their
    scales applied) summed in k order from +0, products rounded then added (a
    plain fp32 model), into leaf g mod 8."""
    lv = np.zeros((8, W.shape[0]), dtype=np.float32)
    for g in range(G):
        p = np.zeros(W.shape[0], dtype=np.float32)
        for t in range(32):
            k = 32 * g + t
            p = (p + (W[:, k] * x[k]).astype(np.float32)).astype(np.float32)
        lv[g % 8] = (lv[g % 8] + p).astype(np.float32)
    return lv


def tree(lv, shape):
    def node(n):
        if isinstance(n, int):
            return lv[n]
        return (node(n[0]) + node(n[1])).astype(np.float32)
    return node(shape)


class Model:
    """CPU model of a gate/up launch over a plan; `plant` names the mistake."""

    def __init__(self, plant=None):
        self.plant = plant
        self.experts = {e: synth.layer_expert(CFG, 0, e) for e in range(CFG.E)}
        self.Wg = {e: oracle.decode_matrix(ex["gate_codes"], ex["gate_scales"]).astype(np.float32)
                   for e, ex in self.experts.items()}
        self.Wu = {e: oracle.decode_matrix(ex["up_codes"], ex["up_scales"]).astype(np.float32)
                   for e, ex in self.experts.items()}

    def plan(self, ids):
        count, offset, entry = oracle.bucket(ids, CFG.E)
        if self.plant == "unstable_bucket":
            rng = np.random.default_rng(int(ids.sum()))
            for e in range(CFG.E):
                a, b = offset[e], offset[e + 1]
                entry[a:b] = rng.permutation(entry[a:b])
        return count, offset, entry, oracle.plan(count, offset, GU_TIERS)

    def run(self, x_bits, logits):
        ids, _ = oracle.route(logits, CFG.k)
        R, k, I = x_bits.shape[0], CFG.k, CFG.I
        x = synth.bf16_bits_to_f32(x_bits)
        _, _, entry, passes = self.plan(ids)
        act = np.full((R * k, I), np.nan, dtype=np.float32)
        for e, first, real, size in passes[::-1]:          # later passes first: a stray write survives
            for r in range(size):
                src = first if self.plant == "first_row" else first + min(r, real - 1)
                row = entry[src] // k
                shape = TREE_SWAPPED if (self.plant == "tree_order" and size > 1) else TREE
                g = tree(leaves(self.Wg[e], x[row], CFG.H // 32), shape)
                u = tree(leaves(self.Wu[e], x[row], CFG.H // 32), shape)
                with np.errstate(over="ignore"):
                    a = (g / (f32(1) + np.exp(-g, dtype=np.float32)) * u).astype(np.float32)
                if r < real:
                    act[entry[first + r]] = a
                elif self.plant == "padding_written" and first + r < R * k:
                    act[entry[first + r]] = a
        return dict(topk_id=ids, entry=entry, act=act.reshape(R, k, I))


def rows_differing(model, x, lg):
    """The probe's check: rows whose act bits differ from the row launched alone."""
    batch = model.run(x, lg)
    bad = 0
    for r in range(x.shape[0]):
        solo = model.run(x[r:r + 1], lg[r:r + 1])
        if not np.array_equal(batch["act"][r].view(np.uint32), solo["act"][0].view(np.uint32)):
            bad += 1
    return bad


def inputs(R, same):
    x = synth.activations(CFG.seed + 31, R, R, CFG.H)
    lg = synth.logits_same(CFG.seed + 31, R, R, CFG.E) if same else synth.logits(CFG.seed + 31, R, R, CFG.E)
    return x, lg


@pytest.fixture(scope="module")
def clean():
    return Model()


@pytest.mark.parametrize("R,same", [(5, True), (9, False)])
def test_unplanted_model_passes_the_probe(clean, R, same):
    x, lg = inputs(R, same)
    assert rows_differing(clean, x, lg) == 0


@pytest.mark.parametrize("plant", ["first_row", "padding_written", "tree_order"])
def test_probe_goes_red_on_planted_mistakes(plant):
    m = Model(plant)
    red = sum(rows_differing(m, *inputs(R, same)) for R, same in ((5, True), (9, False)))
    assert red > 0, plant


def test_tree_order_is_caught_by_bits_not_by_tolerance(clean):
    m = Model("tree_order")
    x, lg = inputs(5, True)
    a, b = m.run(x, lg)["act"], clean.run(x, lg)["act"]
    assert not np.array_equal(a.view(np.uint32), b.view(np.uint32))
    rel = np.abs(a - b).reshape(5, -1).max(axis=1) / np.abs(b).reshape(5, -1).max(axis=1)
    assert np.all(rel <= 1e-3)


def test_plan_check_goes_red_on_unstable_bucketing(clean):
    x, lg = inputs(9, True)                                 # nine rows on the same two experts
    ids, _ = oracle.route(lg, CFG.k)
    want = oracle.bucket(ids, CFG.E)[2]
    assert np.array_equal(clean.run(x, lg)["entry"], want)
    assert not np.array_equal(Model("unstable_bucket").run(x, lg)["entry"], want)
