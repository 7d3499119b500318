"""Pins of the oracle's router variants: correction bias (selection only), the
top-2-sum group score and the route scale (readings R17-R19).

Nothing here runs on a GPU.  Each check is chosen so that a plausible slip (the
bias leaking into the gates, the group rule ignored, the scale applied twice or
dropped from the backward) fails at least one of them.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import moe_oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "router_variants.json")))


def _key(v, idx):
    return (-float(v), int(idx))


def brute_force_topk(v_row, k, n_groups, topk_groups, group_score):
    """Every group subset and every k-subset; the unique dominating one.

    The top-2-sum group score is the largest sum over pairs of distinct
    members, added in the values' own precision.
    """
    E = len(v_row)
    gs = E // n_groups
    gscore = []
    for g in range(n_groups):
        mem = v_row[g * gs:(g + 1) * gs]
        if group_score == "max":
            gscore.append(max(mem))
        else:
            gscore.append(max(mem[a] + mem[b] for a, b in itertools.combinations(range(gs), 2)))
    winners = []
    for G in itertools.combinations(range(n_groups), topk_groups):
        rest = [g for g in range(n_groups) if g not in G]
        if all(_key(gscore[a], a) < _key(gscore[b], b) for a in G for b in rest):
            winners.append(G)
    assert len(winners) == 1
    elig = [e for g in winners[0] for e in range(g * gs, (g + 1) * gs)]
    sets = []
    for S in itertools.combinations(elig, k):
        rest = [e for e in elig if e not in S]
        if all(_key(v_row[a], a) < _key(v_row[b], b) for a in S for b in rest):
            sets.append(S)
    assert len(sets) == 1
    return set(sets[0])


def _values(T, E, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "ties":     # dyadic values on a coarse grid: many exact ties, exact in fp32
        return (rng.integers(0, 6, size=(T, E)) / 8.0).astype(np.float32)
    l = rng.normal(size=(T, E))
    b = (rng.normal(size=E) * 0.05).astype(np.float32)
    return O.selection_values(l, "sigmoid", b, "top2")


CASES = [(4, 2, 2, 1), (6, 3, 3, 2), (8, 2, 4, 2), (8, 3, 2, 1), (8, 5, 4, 3), (8, 2, 4, 1)]


@pytest.mark.parametrize("E,k,G,TG", CASES)
@pytest.mark.parametrize("kind", ["random", "ties"])
@pytest.mark.parametrize("rule", ["max", "top2"])
def test_variant_topk_matches_brute_force(E, k, G, TG, kind, rule):
    v = _values(30, E, kind, seed=E * 97 + k * 13 + G)
    idx = O.select_topk(v, k, G, TG, group_score=rule)
    for t in range(v.shape[0]):
        row = [np.float32(x) for x in v[t]]
        assert set(idx[t].tolist()) == brute_force_topk(row, k, G, TG, rule)
        keys = [_key(v[t, e], e) for e in idx[t]]
        assert keys == sorted(keys)


@pytest.mark.parametrize("rule", ["max", "top2"])
def test_golden_group_rules(rule):
    g = GOLD["group_rules"]
    v = np.array(g["values"], dtype=np.float32)
    idx = O.select_topk(v, g["k"], g["n_groups"], g["topk_groups"], group_score=rule)
    assert idx[0].tolist() == g[rule]["topk_idx"]


def test_golden_bias_selects_and_gates_stay_unbiased():
    g = GOLD["bias"]
    l = np.array(g["logits"])
    b = np.array(g["e_bias"], dtype=np.float32)
    v = O.selection_values(l, "sigmoid", b)
    assert v.dtype == np.float32 and v[0].tolist() == g["values"][0]
    idx = O.select_topk(v, g["k"])
    assert idx[0].tolist() == g["topk_idx_with_bias"]
    gates, _ = O.gate_weights(l, idx, "sigmoid", g["route_scale"])
    assert np.allclose(gates[0], g["gates_with_bias"], rtol=0, atol=1e-15)
    idx0 = O.select_topk(O.selection_values(l, "sigmoid"), g["k"])
    assert idx0[0].tolist() == g["topk_idx_without_bias"]
    gates0, _ = O.gate_weights(l, idx0, "sigmoid", g["route_scale"])
    assert np.allclose(gates0[0], g["gates_without_bias"], rtol=0, atol=1e-15)


def test_zero_bias_max_rule_reduces_to_logit_selection():
    """Sigmoid is increasing: ranking fl32 scores + 0 equals ranking logits when fp32 makes no ties."""
    rng = np.random.default_rng(5)
    l = rng.normal(size=(200, 16))
    v = O.selection_values(l, "sigmoid", np.zeros(16, dtype=np.float32))
    assert v.dtype == np.float32
    rows = [t for t in range(200) if len(set(v[t].tolist())) == 16]
    assert len(rows) > 150
    a = O.select_topk(l[rows], 4, 4, 2)
    b = O.select_topk(v[rows], 4, 4, 2)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("rule", ["max", "top2"])
def test_shift_of_every_value_changes_nothing(rule):
    v = _values(40, 8, "ties", seed=3)
    a = O.select_topk(v, 3, 4, 2, group_score=rule)
    b = O.select_topk((v + np.float32(0.25)).astype(np.float32), 3, 4, 2, group_score=rule)
    assert np.array_equal(a, b)


def test_large_bias_forces_an_expert_and_gates_ignore_the_bias():
    rng = np.random.default_rng(11)
    l = rng.normal(size=(50, 8))
    b = np.zeros(8, dtype=np.float32)
    b[5] = 4.0
    idx = O.select_topk(O.selection_values(l, "sigmoid", b), 2)
    assert np.all(idx[:, 0] == 5)
    g, w = O.gate_weights(l, idx, "sigmoid")
    s = O.sigmoid(l)
    sel = np.take_along_axis(s, idx, axis=1)
    assert np.allclose(g, sel / sel.sum(1, keepdims=True), rtol=1e-15, atol=0)


@pytest.mark.parametrize("c", [1.0, 2.5, 0.5])
def test_route_scale_gates_sum_to_the_scale(c):
    rng = np.random.default_rng(2)
    l = rng.normal(size=(20, 8))
    idx = O.select_topk(l, 3)
    for score in ("softmax", "sigmoid"):
        g, w = O.gate_weights(l, idx, score, c)
        assert np.allclose(g.sum(1), c, rtol=1e-14, atol=0)
        assert np.allclose(g * w.sum(1, keepdims=True), c * w, rtol=1e-14, atol=0)


def _variant_problem(seed):
    rng = np.random.default_rng(seed)
    T, d, ffn, E, k = 10, 4, 5, 8, 2
    b = np.zeros(E, dtype=np.float32)
    b[[1, 6]] = np.float32(0.125)
    shp = O.Shape(E=E, k=k, n_groups=4, topk_groups=2, score="sigmoid", expert="swiglu",
                  group_score="top2", route_scale=2.5)
    for _ in range(500):
        X = rng.normal(size=(T, d))
        P = {"Wg": rng.normal(size=(E, d)), "W1": rng.normal(size=(E, ffn, d)) * 0.5,
             "W2": rng.normal(size=(E, d, ffn)) * 0.5, "W3": rng.normal(size=(E, ffn, d)) * 0.5,
             "e_bias": b}
        v = O.selection_values(X @ P["Wg"].T, "sigmoid", b, "top2").astype(np.float64)
        srt = -np.sort(-v, axis=1)
        top2 = np.sort(v.reshape(T, 4, 2), axis=2).sum(2)
        if (np.all(np.abs(np.diff(srt, axis=1)) > 2e-3)
                and np.all(np.abs(np.diff(-np.sort(-top2, 1), axis=1)) > 2e-3)):
            return X, rng.normal(size=(T, d)), P, shp
    raise RuntimeError("no well-separated draw")


def test_variant_central_differences():
    X, Yt, P, shp = _variant_problem(7)
    aux_coef = 0.3
    st = O.train_step(X, Yt, P, shp, lr=0.0, aux_coef=aux_coef)
    idx = st["fw"]["topk_idx"]
    assert abs(st["fw"]["gates"].sum(1) - 2.5).max() < 1e-12

    def loss():
        fw = O.layer_forward(X, P, shp)
        assert np.array_equal(fw["topk_idx"], idx)
        m, _ = O.mse(fw["Y"], Yt)
        return m + aux_coef * fw["aux"]

    for name, arr in (("dWg", P["Wg"]), ("dX", X), ("dW3", P["W3"])):
        num = np.zeros_like(arr)
        for j in np.ndindex(arr.shape):
            old = arr[j]
            h = 1e-6 * max(1.0, abs(old))
            arr[j] = old + h
            lp = loss()
            arr[j] = old - h
            lm = loss()
            arr[j] = old
            num[j] = (lp - lm) / (2 * h)
        ref = st["grads"][name]
        err = np.abs(num - ref).max() / np.abs(ref).max()
        assert err < 1e-6, (name, err)
