"""Invariants and closed forms of the oracle's whole layer (tiny widths)."""
import numpy as np

import oracle
import synth

CFG = synth.CONFIGS["tiny"]


def _experts(cfg=CFG, layer=0):
    return {e: synth.layer_expert(cfg, layer, e) for e in range(cfg.E)}


def _run(x, lg, ex, cfg=CFG, k=None):
    return oracle.layer(x, lg, ex, cfg.H, cfg.I, cfg.E, k or cfg.k)


def test_zero_activations_give_zero_output():
    x, lg = synth.layer_inputs(CFG)
    res = _run(np.zeros_like(x), lg, _experts())
    assert np.all(res["act"] == 0) and np.all(res["out"] == 0) and np.all(res["y"] == 0)


def test_top1_combine_is_the_expert_output():
    x, lg = synth.layer_inputs(CFG)
    res = _run(x, lg, _experts(), k=1)
    assert np.all(res["topk_w"] == 1.0)
    assert np.array_equal(res["y"], res["out"][:, 0, :])


def test_layer_matches_parts():
    x, lg = synth.layer_inputs(CFG)
    ex = _experts()
    res = _run(x, lg, ex)
    ids, w = oracle.route(lg, CFG.k)
    assert np.array_equal(res["topk_id"], ids) and np.array_equal(res["topk_w"], w)
    xf = oracle.bf16_to_f64(x)
    for r in range(CFG.R):
        for j in range(CFG.k):
            e = ex[int(ids[r, j])]
            g = oracle.matvec(e["gate_codes"], e["gate_scales"], xf[r])
            u = oracle.matvec(e["up_codes"], e["up_scales"], xf[r])
            a = oracle.swiglu(g, u)
            assert np.array_equal(res["act"][r, j], a)
            assert np.array_equal(res["out"][r, j], oracle.matvec(e["down_codes"], e["down_scales"], a))
        assert np.array_equal(res["y"][r], oracle.combine(w[r], res["out"][r]))


def test_row_permutation_and_duplicates():
    x, lg = synth.layer_inputs(CFG)
    ex = _experts()
    base = _run(x, lg, ex)
    perm = np.array([2, 0, 3, 1])
    p = _run(x[perm], lg[perm], ex)
    for name in ("act", "out", "y", "topk_id", "topk_w"):
        assert np.array_equal(p[name], base[name][perm]), name
    dup = _run(np.repeat(x[:1], 3, axis=0), np.repeat(lg[:1], 3, axis=0), ex)
    assert np.array_equal(dup["y"][0], dup["y"][1]) and np.array_equal(dup["y"][0], dup["y"][2])
    assert np.array_equal(dup["y"][0], base["y"][0])


def test_expert_relabelling_leaves_output_unchanged():
    x, lg = synth.layer_inputs(CFG)
    ex = _experts()
    base = _run(x, lg, ex)
    sigma = np.array([5, 2, 7, 0, 1, 6, 3, 4])           # new id of old expert e is sigma[e]
    ex2 = {int(sigma[e]): ex[e] for e in ex}
    lg2 = np.empty_like(lg)
    lg2[:, sigma] = lg
    res = _run(x, lg2, ex2)
    assert np.array_equal(res["topk_id"], sigma[base["topk_id"]])
    assert np.array_equal(res["y"], base["y"])


def test_nan_and_inf_stay_in_their_rows():
    cfg = synth.CONFIGS["tiny"]
    x, lg = synth.layer_inputs(cfg)
    xp, (nr, _), (ir, _) = synth.plant_nan_inf(cfg.seed, 0, x)
    res = _run(xp, lg, _experts())
    clean = _run(x, lg, _experts())
    for r in range(cfg.R):
        if r in (nr, ir):
            assert not np.all(np.isfinite(res["y"][r]))
        else:
            assert np.array_equal(res["y"][r], clean["y"][r])
    assert np.all(np.isnan(res["act"][nr]))
