"""moe_route_noalloc (routing with the scratch in the library's static device array)
against moe_route (the same kernels with the scratch in the caller's workspace).

Two calls in a row on the same GPU, the second with fewer tokens, each compared
bit for bit with moe_route on the same logits; the routing is also checked
against the oracle's selection on those logits.  The array keeps the first
call's contents when the second runs, so this also shows that nothing is read
before it is written.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from sparse_mixture_experts_gate_amd import _lib as L
from sparse_mixture_experts_gate_amd import workloads as W

pytestmark = pytest.mark.gpu


def _workload(T, E, k, G, TG, score, **kw):
    return W.Workload("route", T=T, d=64, E=E, ffn=64, k=k, n_groups=G, topk_groups=TG, score=score,
                      expert="swiglu", dtype="bf16", lr=0.0, aux_coef=0.0, steps=1, init="fan_in",
                      gate="normal", **kw)


def _with_workspace(w, logits, bias):
    cfg = L.config(w)
    ws = L.alloc_workspace(cfg, "cuda")
    r = L.alloc_routing(w, "cuda")
    L.moe_route(cfg, logits, r, ws, e_bias=bias)
    torch.cuda.synchronize()
    return {n: v.cpu() for n, v in r.items() if n != "logits"}


def _no_alloc(w, logits, bias):
    cfg = L.config(w)
    r = L.alloc_routing(w, "cuda")
    L.moe_route_noalloc(cfg, logits, r, e_bias=bias)
    torch.cuda.synchronize()
    return {n: v.cpu() for n, v in r.items() if n != "logits"}


@pytest.mark.parametrize("E,k,G,TG,score,bias,gs", [
    (256, 8, 8, 4, "sigmoid", 0.0, "max"),
    (64, 6, 8, 4, "sigmoid", 0.1, "top2"),
    (8, 2, 1, 1, "softmax", 0.0, "max"),
])
def test_noalloc_route_equals_route(E, k, G, TG, score, bias, gs):
    for T in (20000, 777):                      # the second call is smaller
        w = _workload(T, E, k, G, TG, score, e_bias=bias, group_score=gs)
        logits = W.make_router_logits(T, E, "normal", seed=T + E).cuda()
        b = W.make_inputs(w.replace(T=1), seed=T)["e_bias"]
        b = None if b is None else b.cuda()
        ref = _with_workspace(w, logits, b)
        got = _no_alloc(w, logits, b)
        assert ref.keys() == got.keys()
        for n in ref:
            assert torch.equal(ref[n], got[n]), (T, n)
        l64 = logits.double().cpu().numpy()
        v = O.selection_values(l64, score, None if b is None else b.cpu().numpy(), gs)
        sel = O.select_topk(v, k, G, TG, group_score=gs)
        assert np.array_equal(got["topk_idx"].numpy(), sel), T
        rt = O.routing_tables(sel, E)
        assert np.array_equal(got["slot_of"].numpy(), rt.slot_of), T
        assert np.array_equal(got["offsets"].numpy(), rt.offsets), T
