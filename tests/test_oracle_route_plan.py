"""Pins of the oracle's routing, bucketing and pass plan (brute force, invariants, the pages' worked example)."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth


def _brute_topk(row, k):
    def key(e):
        v = float(row[e])
        return (1, 0.0, e) if math.isnan(v) else (0, -v, e)
    return sorted(range(len(row)), key=key)[:k]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_topk_matches_sort(seed):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((9, 40)).astype(np.float32)
    lg[0, 3] = lg[0, 7] = lg[0, 11] = 5.0          # ties -> lower id first
    lg[1, :] = np.nan                              # all NaN -> ids ascending
    lg[2, 5] = np.nan
    lg[2, 6] = -np.inf
    lg[3, :5] = np.inf
    lg[4, 10] = -0.0
    lg[4, 2] = 0.0
    ids, w = oracle.route(lg, 6)
    for r in range(lg.shape[0]):
        assert list(ids[r]) == _brute_topk(lg[r], 6), r
    assert list(ids[0][:3]) == [3, 7, 11]
    assert list(ids[1]) == [0, 1, 2, 3, 4, 5]


def test_softmax_weights_closed_form():
    lg = np.array([[0.0, math.log(2.0), math.log(4.0), -50.0]], dtype=np.float32)
    ids, w = oracle.route(lg, 3)
    assert list(ids[0]) == [2, 1, 0]
    want = np.array([4, 2, 1], dtype=np.float64) / 7.0
    l = lg[0][[2, 1, 0]].astype(np.float64)
    exact = np.exp(l - l.max()) / np.exp(l - l.max()).sum()
    assert np.allclose(w[0], exact, rtol=1e-15, atol=0)
    assert np.allclose(w[0], want, rtol=1e-6)
    # k = 1 -> weight exactly 1
    _, w1 = oracle.route(lg, 1)
    assert w1[0, 0] == 1.0


def test_softmax_properties_random():
    lg = synth.logits(5, 0, 16, 256)
    ids, w = oracle.route(lg, 8)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)       # slots ordered by descending logit
    for r in range(16):
        l = lg[r, ids[r]].astype(np.float64)
        assert np.allclose(np.log(w[r, 0] / w[r, 1:]), l[0] - l[1:], rtol=0, atol=1e-12)


def _brute_bucket(ids, E):
    R, k = ids.shape
    pairs = sorted(((int(ids[r, j]), r, r * k + j) for r in range(R) for j in range(k)))
    entry = [p[2] for p in pairs]
    count = [sum(1 for p in pairs if p[0] == e) for e in range(E)]
    return count, entry


@pytest.mark.parametrize("R,E,k", [(1, 8, 2), (4, 8, 2), (16, 256, 8), (37, 64, 6), (3, 3, 3)])
def test_bucket_matches_sort(R, E, k):
    lg = synth.logits(11, R, R, E)
    ids, _ = oracle.route(lg, k)
    count, offset, entry = oracle.bucket(ids, E)
    bc, be = _brute_bucket(ids, E)
    assert list(count) == bc
    assert list(entry) == be
    assert offset[0] == 0 and list(np.diff(offset)) == bc


def _golden_passes(golden_dir):
    with open(os.path.join(golden_dir, "pass_sizes.json")) as f:
        return json.load(f)


def test_pass_sizes_worked_example(golden_dir):
    g = _golden_passes(golden_dir)
    for case in g["cases"]:
        got_gu = [list(p) for p in oracle.passes(case["rows"], g["tiers"]["gateup"])]
        got_dn = [list(p) for p in oracle.passes(case["rows"], g["tiers"]["down"])]
        assert got_gu == case["gateup"], case
        assert got_dn == case["down"], case


# hand table from the pass rule (size, real) for gate/up {2,4,6,8} | down {2,4}
HAND = {
    2: ([(2, 2)], [(2, 2)]),
    3: ([(4, 3)], [(4, 3)]),
    4: ([(4, 4)], [(4, 4)]),
    5: ([(6, 5)], [(4, 4), (2, 1)]),
    6: ([(6, 6)], [(4, 4), (2, 2)]),
    7: ([(8, 7)], [(4, 4), (4, 3)]),
    8: ([(8, 8)], [(4, 4), (4, 4)]),
    9: ([(8, 8), (2, 1)], [(4, 4), (4, 4), (2, 1)]),
    16: ([(8, 8), (8, 8)], [(4, 4)] * 4),
}


@pytest.mark.parametrize("n", sorted(HAND))
def test_pass_hand_table(n):
    gu, dn = HAND[n]
    assert oracle.passes(n, [2, 4, 6, 8]) == gu
    assert oracle.passes(n, [2, 4]) == dn


@pytest.mark.parametrize("tiers", [[2, 4, 6, 8], [2, 4], [4], [8], [2, 4, 8], [2, 3, 5, 7, 8]])
def test_pass_rule_properties(tiers):
    for n in range(1, 33):
        ps = oracle.passes(n, tiers)
        assert sum(r for _, r in ps) == n
        if n == 1:
            assert ps == [(1, 1)]
            continue
        for i, (p, r) in enumerate(ps):
            assert p in tiers and 1 <= r <= p
            if i < len(ps) - 1:
                assert r == p == max(tiers)        # only the last pass may pad
        # the last pass is the smallest size that holds what is left
        p, r = ps[-1]
        assert p == min(t for t in tiers if t >= r) or (r == max(tiers) == p)


def test_plan_layout_matches_passes():
    lg = synth.logits(3, 0, 16, 32)
    ids, _ = oracle.route(lg, 8)
    count, offset, entry = oracle.bucket(ids, 32)
    plan = oracle.plan(count, offset, [2, 4, 6, 8])
    # experts ascending, passes tile each expert's entries in order
    pos = {}
    for e, first, real, size in plan:
        assert first == pos.get(e, offset[e])
        pos[e] = first + real
    for e in range(32):
        assert pos.get(e, offset[e]) == offset[e + 1]
    assert list(plan[:, 0]) == sorted(plan[:, 0])


def test_plan_for_an_expert_with_many_rows():
    # 1000 rows on one expert: 125 passes of 8 (gate/up), 250 of 4 (down)
    count = np.array([1000, 0, 3], dtype=np.int32)
    offset = np.array([0, 1000, 1000, 1003], dtype=np.int32)
    gu = oracle.plan(count, offset, [2, 4, 6, 8])
    assert len(gu) == 126 and np.all(gu[:125, 3] == 8) and np.all(gu[:125, 2] == 8)
    assert list(gu[125]) == [2, 1000, 3, 4]
    assert list(gu[:125, 1]) == list(range(0, 1000, 8))
    dn = oracle.plan(count, offset, [2, 4])
    assert len(dn) == 251 and list(dn[-1]) == [2, 1000, 3, 4] and np.all(dn[:250, 3] == 4)
