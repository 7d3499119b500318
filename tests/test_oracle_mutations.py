"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in the oracle (on the CPU, by monkeypatching one
function) and asserts that at least one pin test then fails.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O

import tests.test_oracle_layer as L
import tests.test_oracle_routing as R
import tests.test_oracle_shared as S
import tests.test_oracle_variants as V


def _larger_id_wins(l, k, n_groups=1, topk_groups=1, **kw):
    # tie rule flipped: among equal logits the larger id comes first
    T, E = l.shape
    idx = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        order = np.lexsort((-np.arange(E), -l[t]))
        idx[t] = order[:k]
    return idx


def _no_renorm(l, topk_idx, score, route_scale=1.0):
    w = np.take_along_axis(O.scores(l, score), topk_idx, axis=1)
    return w, w


def _aux_over_T(counts, q, k):
    T, E = q.shape
    f = counts / float(T)
    P = q.mean(axis=0)
    return E * float(np.dot(f, P)), f, P


def _sigmoid_unnormalised(l, score):
    return O.scores(l, score)


def _bad_silu_grad(x):
    s = O.sigmoid(x)
    return s * (1.0 + x * s)


def _descending_slots(topk_idx, E):
    r = _orig_tables(topk_idx[::-1], E)
    T, k = topk_idx.shape
    return O.Routing(topk_idx, r.counts, r.offsets, r.slot_of[::-1], (T - 1) - r.token_of, r.src_k)


_orig_tables = O.routing_tables
_orig_router_backward = O.router_backward


def _router_backward_wrong_sign(l, topk_idx, dw, dq, score):
    return -_orig_router_backward(l, topk_idx, dw, dq, score)


_orig_select = O.select_topk


def _orig_select_min(l, k, n_groups=1, topk_groups=1, **kw):
    T, E = l.shape
    gsize = E // n_groups
    gscore = l.reshape(T, n_groups, gsize).min(axis=2)
    kept = np.zeros((T, n_groups), dtype=bool)
    for t in range(T):
        kept[t, np.lexsort((np.arange(n_groups), -gscore[t]))[:topk_groups]] = True
    elig = np.repeat(kept, gsize, axis=1)
    idx = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        idx[t] = np.lexsort((np.arange(E), -l[t], ~elig[t]))[:k]
    return idx


_orig_selection_values = O.selection_values
_orig_gate_weights = O.gate_weights
_orig_renorm_backward = O.renorm_backward


def _bias_ignored(l, score, e_bias=None, group_score="max"):
    return _orig_selection_values(l, score, None, "top2" if e_bias is not None else group_score)


def _group_rule_ignored(l, k, n_groups=1, topk_groups=1, group_score="max"):
    return _orig_select(l, k, n_groups, topk_groups)


def _scale_dropped(l, topk_idx, score, route_scale=1.0):
    return _orig_gate_weights(l, topk_idx, score, 1.0)


def _scale_missing_in_backward(dgate, gates, w, route_scale=1.0):
    return _orig_renorm_backward(dgate, gates, w, 1.0)


_orig_shared_backward = O.shared_backward


def _shared_roles_swapped(X, P):
    # gate and up projections exchanged: A = silu(X Ws3^T) * (X Ws1^T)
    return O.expert_forward("swiglu", X, P["Ws3"], None, P["Ws2"], None, P["Ws1"])


def _shared_dx_dropped(X, P, saved, dY):
    g = _orig_shared_backward(X, P, saved, dY)
    g["dX"] = np.zeros_like(g["dX"])
    return g


def _shared_half_gradient(X, P, saved, dY):
    # upstream gradient scaled as if the branch carried a gate of 1/2
    return _orig_shared_backward(X, P, saved, 0.5 * dY)


def _run_all(fns):
    failed = 0
    for fn, args in fns:
        try:
            fn(*args)
        except (AssertionError, ValueError, IndexError, TypeError):
            failed += 1
    return failed


PINS = [
    (R.test_topk_matches_brute_force, (8, 2, 4, 2, "ties")),
    (R.test_topk_matches_brute_force, (6, 3, 2, 1, "ties")),
    (R.test_signed_zero_ties_go_to_smaller_id, ()),
    (R.test_group_limit_excludes_a_large_logit_in_a_dropped_group, ()),
    (R.test_gates_closed_forms_softmax, ()),
    (R.test_routing_tables_definition, (33, 8, 3)),
    (R.test_aux_is_one_under_uniform_routing, ("softmax", 64, 8, 3, 1, 1)),
    (R.test_aux_is_one_under_uniform_routing, ("sigmoid", 64, 8, 3, 1, 1)),
    (L.test_hand_worked_golden, ()),
    (L.test_central_differences, ("swiglu", "sigmoid", 1)),
    (L.test_central_differences, ("gelu", "softmax", 2)),
    (V.test_variant_topk_matches_brute_force, (8, 2, 4, 2, "ties", "top2")),
    (V.test_golden_group_rules, ("top2",)),
    (V.test_golden_bias_selects_and_gates_stay_unbiased, ()),
    (V.test_route_scale_gates_sum_to_the_scale, (2.5,)),
    (V.test_variant_central_differences, ()),
    (S.test_shared_branch_is_one_routed_expert_over_every_token, ("swiglu",)),
    (S.test_shared_central_differences, ("swiglu",)),
    (S.test_zero_output_projection_and_linearity, ()),
]


@pytest.mark.parametrize("name,repl", [
    ("select_topk", _larger_id_wins),
    ("select_topk", _orig_select_min),
    ("gate_weights", _no_renorm),
    ("aux_loss", _aux_over_T),
    ("aux_probs", _sigmoid_unnormalised),
    ("silu_grad", _bad_silu_grad),
    ("routing_tables", _descending_slots),
    ("router_backward", _router_backward_wrong_sign),
    ("selection_values", _bias_ignored),
    ("select_topk", _group_rule_ignored),
    ("gate_weights", _scale_dropped),
    ("renorm_backward", _scale_missing_in_backward),
    ("shared_forward", _shared_roles_swapped),
    ("shared_backward", _shared_dx_dropped),
    ("shared_backward", _shared_half_gradient),
])
def test_planted_mistake_is_caught(monkeypatch, name, repl):
    monkeypatch.setattr(O, name, repl)
    assert _run_all(PINS) >= 1, f"no pin caught a mistake planted in {name}"
