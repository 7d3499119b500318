"""Pins of the oracle's routing steps against brute force, closed forms and invariants.

Nothing here runs on a GPU.  Each check is chosen so that a plausible slip in
the oracle (a flipped tie rule, a wrong group block, a sort on the wrong key,
an off-by-one in the scan, a missing normalisation) fails it.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from sparse_mixture_experts_gate_amd import workloads as W


def _key(v, idx):
    # (-value, id): Python compares -0.0 == 0.0, so the id decides such ties.
    return (-float(v), int(idx))


def brute_force_topk(l_row, k, n_groups, topk_groups):
    """Enumerate every group subset and every k-subset; keep the unique dominating one."""
    E = len(l_row)
    gs = E // n_groups
    gscore = [max(l_row[g * gs:(g + 1) * gs]) for g in range(n_groups)]
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
        if all(_key(l_row[a], a) < _key(l_row[b], b) for a in S for b in rest):
            sets.append(S)
    assert len(sets) == 1
    return set(sets[0])


CASES = [(4, 2, 1, 1), (4, 1, 1, 1), (4, 4, 1, 1), (6, 3, 2, 1), (8, 2, 4, 2), (8, 3, 2, 1),
         (8, 5, 4, 3), (8, 8, 1, 1), (8, 2, 8, 2)]


@pytest.mark.parametrize("E,k,G,TG", CASES)
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_topk_matches_brute_force(E, k, G, TG, kind):
    if k > TG * (E // G):
        pytest.skip("k larger than the eligible experts")
    l = W.make_router_logits(40, E, kind, seed=E * 100 + k * 10 + G).double().numpy()
    idx = O.select_topk(l, k, G, TG)
    for t in range(l.shape[0]):
        assert set(idx[t].tolist()) == brute_force_topk(l[t].tolist(), k, G, TG)
        keys = [_key(l[t, e], e) for e in idx[t]]
        assert keys == sorted(keys), "output not in (-logit, id) order"
        assert len(set(idx[t].tolist())) == k


def test_signed_zero_ties_go_to_smaller_id():
    l = np.array([[-0.0, 0.0, -1.0, 0.0], [0.0, -0.0, 0.0, -0.0]])
    assert O.select_topk(l, 2).tolist() == [[0, 1], [0, 1]]
    assert O.select_topk(l, 3).tolist() == [[0, 1, 3], [0, 1, 2]]


def test_group_limit_excludes_a_large_logit_in_a_dropped_group():
    # group 0 = {0,1}, group 1 = {2,3}, group 2 = {4,5}; keep 2 groups.
    # Group scores: 5, 4, 4.5 -> keep groups 0 and 2; expert 2 (logit 4) is
    # dropped although it beats expert 1 (logit 0).
    l = np.array([[5.0, 0.0, 4.0, -9.0, 4.5, 1.0]])
    assert O.select_topk(l, 3, n_groups=3, topk_groups=2).tolist() == [[0, 4, 5]]
    # equal group scores: the smaller group id is kept
    l = np.array([[1.0, 0.0, 1.0, 0.5, 0.0, 2.0]])
    assert O.select_topk(l, 2, n_groups=3, topk_groups=2).tolist() == [[5, 0]]


def test_gates_closed_forms_softmax():
    l = W.make_router_logits(50, 8, "normal", seed=3).double().numpy()
    idx = O.select_topk(l, 3)
    g, w = O.gate_weights(l, idx, "softmax")
    for t in range(50):
        sel = [l[t, e] for e in idx[t]]
        z = [math.exp(v - max(sel)) for v in sel]
        want = [v / sum(z) for v in z]          # softmax over the selected logits
        assert np.allclose(g[t], want, rtol=1e-13, atol=0)
        assert abs(g[t].sum() - 1.0) < 4 * np.finfo(float).eps
        assert np.all(g[t] > 0) and np.all(g[t] <= 1)
    p = O.scores(l, "softmax")
    idxE = O.select_topk(l, 8)
    gE, _ = O.gate_weights(l, idxE, "softmax")
    assert np.allclose(gE, np.take_along_axis(p, idxE, 1), rtol=1e-13)   # k = E: g = p
    g1, _ = O.gate_weights(l, O.select_topk(l, 1), "softmax")
    assert np.all(g1 == 1.0)                                              # k = 1: g = 1


def test_gates_closed_forms_sigmoid():
    l = W.make_router_logits(30, 8, "normal", seed=4).double().numpy()
    idx = O.select_topk(l, 4, 4, 2)
    g, w = O.gate_weights(l, idx, "sigmoid")
    for t in range(30):
        s = [1.0 / (1.0 + math.exp(-l[t, e])) for e in idx[t]]
        assert np.allclose(g[t], [v / sum(s) for v in s], rtol=1e-13, atol=0)
        assert np.allclose(w[t], s, rtol=1e-14)


def test_softmax_rows_matches_definition():
    l = np.array([[1000.0, 999.0, -5.0], [0.0, 0.0, 0.0]])
    p = O.softmax_rows(l)
    e1 = math.exp(-1.0)
    e6 = math.exp(-1005.0)
    assert np.allclose(p[0], [1 / (1 + e1 + e6), e1 / (1 + e1 + e6), e6 / (1 + e1 + e6)], rtol=1e-14)
    assert np.allclose(p[1], [1 / 3] * 3, rtol=1e-15)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 4, 2), (33, 8, 3), (64, 16, 16), (5, 6, 1)])
def test_routing_tables_definition(T, E, k):
    l = W.make_router_logits(T, E, "ties", seed=T + E + k).double().numpy()
    idx = O.select_topk(l, k)
    r = O.routing_tables(idx, E)
    assert r.counts.sum() == T * k
    assert r.offsets[0] == 0 and np.all(np.diff(r.offsets) == r.counts)
    for t in range(T):
        for i in range(k):
            e = idx[t, i]
            before = sum(1 for tp in range(t) if e in idx[tp])
            assert r.slot_of[t, i] == r.offsets[e] + before
    assert sorted(r.slot_of.reshape(-1).tolist()) == list(range(T * k))
    for t in range(T):
        for i in range(k):
            assert r.token_of[r.slot_of[t, i]] == t
            assert r.src_k[r.slot_of[t, i]] == i
    for p in range(T * k):                      # brute force: the unique (t, i) stored at row p
        hits = [(t, i) for t in range(T) for i in range(k) if r.slot_of[t, i] == p]
        assert hits == [(r.token_of[p], r.src_k[p])]
    for e in range(E):
        seg = r.token_of[r.offsets[e]:r.offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_empty_expert_segments():
    idx = np.array([[2, 0], [0, 2], [2, 0]])
    r = O.routing_tables(idx, 5)
    assert r.counts.tolist() == [3, 0, 3, 0, 0]
    assert r.offsets.tolist() == [0, 3, 3, 6, 6, 6]
    assert r.slot_of.tolist() == [[3, 0], [1, 4], [5, 2]]
    assert r.token_of.tolist() == [0, 1, 2, 0, 1, 2]
    assert r.src_k.tolist() == [1, 0, 1, 0, 1, 0]


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("T,E,k,G,TG", [(8, 4, 2, 1, 1), (64, 8, 3, 1, 1), (32, 16, 4, 4, 2),
                                        (256, 64, 6, 8, 4)])
def test_aux_is_one_under_uniform_routing(score, T, E, k, G, TG):
    l = W.make_router_logits(T, E, "uniform").double().numpy()
    idx = O.select_topk(l, k, G, TG)
    r = O.routing_tables(idx, E)
    assert np.all(r.counts == T * k // E)
    aux, f, P = O.aux_loss(r.counts, O.aux_probs(l, score), k)
    assert abs(aux - 1.0) < 1e-12
    assert np.allclose(P, 1.0 / E, atol=1e-14)


def test_aux_values_on_skewed_routing():
    # Every token picks expert 0 (k=1): f = (1,0,..), aux = E * P_0 >= 1.
    l = np.array([[3.0, 0.0, 0.0, 0.0]] * 4)
    r = O.routing_tables(O.select_topk(l, 1), 4)
    aux, f, P = O.aux_loss(r.counts, O.aux_probs(l, "softmax"), 1)
    p0 = math.exp(3) / (math.exp(3) + 3)
    assert abs(aux - 4 * p0) < 1e-14


def test_aux_probs_sigmoid_normalised():
    l = W.make_router_logits(10, 6, "normal", seed=9).double().numpy()
    q = O.aux_probs(l, "sigmoid")
    s = 1 / (1 + np.exp(-l))
    assert np.allclose(q, s / s.sum(1, keepdims=True), rtol=1e-15)
    assert np.allclose(q.sum(1), 1.0, rtol=1e-15)


def test_workload_generator_skewed_gate_leaves_three_experts_empty():
    w = W.BY_NAME["skewed_swiglu_t8192_e32"]
    Wg = W.make_gate(w).to(torch.bfloat16)
    assert torch.equal(Wg[25], Wg[31]) and torch.equal(Wg[26], Wg[30])
    X = W.make_inputs(w.replace(T=512, d=w.d, E=w.E, ffn=64))["X"]
    l = (X.double() @ Wg.double().T).numpy()
    idx = O.select_topk(l, w.k)
    counts = O.routing_tables(idx, w.E).counts
    assert counts[29] == counts[30] == counts[31] == 0
