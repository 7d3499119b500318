"""Routing through moe_route is bit-exact against the oracle on identical logits.

The logits are seeded inputs (normal, tie-heavy with +/-0.0, and perfectly
uniform cyclic shifts), so top-k, counts, offsets and slot maps must match
the oracle exactly; gates and aux are fp32 results compared at relative 1e-5.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from sparse_mixture_experts_gate_amd import _lib as L
from sparse_mixture_experts_gate_amd import workloads as W
from tests.gpu_harness import assert_close, say

pytestmark = pytest.mark.gpu

CASES = [
    # T, E, k, G, TG, score, kind
    (1000, 8, 2, 1, 1, "softmax", "normal"),
    (1000, 8, 2, 1, 1, "softmax", "ties"),
    (777, 64, 6, 8, 4, "sigmoid", "normal"),
    (777, 64, 6, 8, 4, "sigmoid", "ties"),
    (300, 256, 8, 8, 4, "sigmoid", "normal"),
    (300, 256, 8, 8, 4, "sigmoid", "ties"),
    (129, 32, 4, 1, 1, "softmax", "ties"),
    (64, 4, 2, 1, 1, "softmax", "normal"),
    (65, 16, 16, 1, 1, "softmax", "normal"),       # k = E
    (100, 8, 1, 1, 1, "sigmoid", "normal"),        # k = 1
    (200, 256, 16, 128, 8, "softmax", "normal"),   # 128 groups of two
    (130, 10, 3, 5, 2, "softmax", "ties"),
    (1, 8, 3, 2, 1, "sigmoid", "normal"),
    (0, 8, 2, 1, 1, "softmax", "normal"),          # no tokens
]


def _workload(T, E, k, G, TG, score, **kw):
    return W.Workload("route", T=T, d=4, E=E, ffn=4, k=k, n_groups=G, topk_groups=TG, score=score,
                      expert="relu", dtype="f32", lr=0.0, aux_coef=0.0, steps=1, init="fan_in",
                      gate="normal", **kw)


def _route(w, logits, e_bias=None):
    cfg = L.config(w)
    ws = L.alloc_workspace(cfg, "cuda")
    r = L.alloc_routing(w, "cuda")
    L.moe_route(cfg, logits.cuda(), r, ws, e_bias=None if e_bias is None else e_bias.cuda())
    torch.cuda.synchronize()
    return {n: v.cpu() for n, v in r.items()}


@pytest.mark.parametrize("T,E,k,G,TG,score,kind", CASES)
def test_route_bit_exact(T, E, k, G, TG, score, kind):
    say(f"route T={T} E={E} k={k} G={G}/{TG} {score} {kind}")
    w = _workload(T, E, k, G, TG, score)
    logits = W.make_router_logits(T, E, kind, seed=T + E)
    r = _route(w, logits)
    l64 = logits.double().numpy()
    ref = O.select_topk(l64, k, G, TG) if T else np.zeros((0, k), dtype=np.int64)
    assert np.array_equal(r["topk_idx"].numpy(), ref)
    rt = O.routing_tables(ref, E)
    assert np.array_equal(r["counts"].numpy(), rt.counts)
    assert np.array_equal(r["offsets"].numpy(), rt.offsets)
    assert np.array_equal(r["slot_of"].numpy(), rt.slot_of)
    assert np.array_equal(r["token_of"].numpy(), rt.token_of)
    assert np.array_equal(r["src_k"].numpy(), rt.src_k)
    if T:
        g, _ = O.gate_weights(l64, ref, score)
        assert_close("gates", r["gates"].double().numpy(), g, 1e-5, 1e-5)
        aux, _, _ = O.aux_loss(rt.counts, O.aux_probs(l64, score), k)
        assert_close("aux", r["aux"].double().numpy(), [aux], 1e-5, 1e-5)
    else:
        assert float(r["aux"][0]) == 0.0


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_route_uniform_gives_aux_one(score):
    w = _workload(640, 64, 6, 8, 4, score)
    r = _route(w, W.make_router_logits(640, 64, "uniform"))
    assert np.all(r["counts"].numpy() == 640 * 6 // 64)
    assert abs(float(r["aux"][0]) - 1.0) < 1e-5


def test_route_is_deterministic():
    w = _workload(5000, 256, 8, 8, 4, "sigmoid")
    logits = W.make_router_logits(5000, 256, "ties", seed=3)
    a, b = _route(w, logits), _route(w, logits)
    for n in a:
        assert torch.equal(a[n], b[n]), n


# router variants: (T, E, k, G, TG, score, kind, bias std, group score, route scale)
VARIANTS = [
    (777, 64, 6, 8, 4, "sigmoid", "normal", 0.1, "top2", 2.5),
    (300, 256, 8, 8, 4, "sigmoid", "ties", 0.25, "top2", 1.0),
    (500, 32, 4, 4, 2, "softmax", "normal", 0.0, "top2", 1.0),
    (400, 64, 6, 8, 4, "sigmoid", "normal", 0.1, "max", 1.0),
    (256, 256, 8, 128, 16, "sigmoid", "normal", 0.05, "top2", 0.5),   # 128 groups of two
    (0, 8, 2, 2, 1, "sigmoid", "normal", 0.1, "top2", 2.0),           # no tokens
]


@pytest.mark.parametrize("T,E,k,G,TG,score,kind,bstd,gs,rs", VARIANTS)
def test_route_variants(T, E, k, G, TG, score, kind, bstd, gs, rs):
    """Bit-exact on identical logits: the oracle ranks the fp32 rounding of its float64
    scores plus the fp32 bias, and so does the kernel (scores evaluated in float64)."""
    say(f"route variant T={T} E={E} k={k} G={G}/{TG} {score} {kind} bias={bstd} {gs} scale={rs}")
    w = _workload(T, E, k, G, TG, score, group_score=gs, route_scale=rs, e_bias=bstd)
    logits = W.make_router_logits(T, E, kind, seed=T + E + 1)
    bias = W.make_inputs(w.replace(T=1, d=8, ffn=8), seed=T)["e_bias"]
    r = _route(w, logits, bias)
    l64 = logits.double().numpy()
    b32 = None if bias is None else bias.numpy().astype(np.float32)
    if T == 0:
        assert float(r["aux"][0]) == 0.0
        return
    v = O.selection_values(l64, score, b32, gs)
    ref = O.select_topk(v, k, G, TG, group_score=gs)
    n_diff = int(np.any(r["topk_idx"].numpy() != ref, axis=1).sum())
    assert n_diff == 0, f"{n_diff} of {T} tokens select differently"
    rt = O.routing_tables(ref, E)
    assert np.array_equal(r["counts"].numpy(), rt.counts)
    assert np.array_equal(r["offsets"].numpy(), rt.offsets)
    assert np.array_equal(r["slot_of"].numpy(), rt.slot_of)
    assert np.array_equal(r["token_of"].numpy(), rt.token_of)
    assert np.array_equal(r["src_k"].numpy(), rt.src_k)
    g, _ = O.gate_weights(l64, ref, score, rs)
    assert_close("gates", r["gates"].double().numpy(), g, 1e-5, 1e-5)
    aux, _, _ = O.aux_loss(rt.counts, O.aux_probs(l64, score), k)
    assert_close("aux", r["aux"].double().numpy(), [aux], 1e-5, 1e-5)


def test_bias_changes_picks_but_not_the_gates_of_unchanged_picks():
    w0 = _workload(2000, 64, 6, 8, 4, "sigmoid")
    wb = w0.replace(e_bias=0.01)          # small enough to leave about a quarter of the picks
    logits = W.make_router_logits(2000, 64, "normal", seed=9)
    bias = W.make_inputs(wb.replace(T=1, d=8, ffn=8), seed=4)["e_bias"]
    a = _route(w0, logits)
    b = _route(wb, logits, bias)
    same = np.all(a["topk_idx"].numpy() == b["topk_idx"].numpy(), axis=1)
    assert 0 < same.sum() < 2000, "the bias should change some picks and leave others"
    assert torch.equal(a["gates"][same], b["gates"][same])


def test_src_k_is_optional():
    """With src_k NULL every other routing output is the same as with it."""
    w = _workload(777, 64, 6, 8, 4, "sigmoid")
    logits = W.make_router_logits(777, 64, "normal", seed=5)
    full = _route(w, logits)
    cfg = L.config(w)
    ws = L.alloc_workspace(cfg, "cuda")
    r = L.alloc_routing(w, "cuda")
    r.pop("src_k")
    L.moe_route(cfg, logits.cuda(), r, ws)
    torch.cuda.synchronize()
    for n, v in r.items():
        if n != "logits":
            assert torch.equal(v.cpu(), full[n]), n
