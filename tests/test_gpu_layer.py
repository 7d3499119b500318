"""Whole-layer parity of the HIP path against the float64 oracle on small shapes.

Shapes are small enough for the oracle to finish in seconds but span several
MFMA tiles in every dimension with ragged tails (256-row / 256-column tiles,
64-deep k steps), and cover the degenerate cases: an expert with no rows,
k = 1, k = E, one token, no tokens.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from sparse_mixture_experts_gate_amd import _lib as L
from sparse_mixture_experts_gate_amd import workloads as W
from tests.gpu_harness import (TOL, LayerRun, assert_close, check_routing, full_parity, oracle_params,
                               say, shape_of, to64)

pytestmark = pytest.mark.gpu


def wl(name, **kw):
    base = dict(T=100, d=32, E=8, ffn=48, k=2, n_groups=1, topk_groups=1, score="softmax",
                expert="relu", dtype="f32", lr=1e-2, aux_coef=0.01, steps=1, init="fan_in",
                gate="normal")
    base.update(kw)
    return W.Workload(name, **base)


F32_CASES = [
    wl("f32_relu_softmax"),
    wl("f32_gelu_softmax", expert="gelu"),
    wl("f32_swiglu_sigmoid_groups", expert="swiglu", score="sigmoid", n_groups=2, topk_groups=1),
    wl("f32_gelu_sigmoid", expert="gelu", score="sigmoid", E=6, k=3),
    wl("f32_relu_k1", k=1),
    wl("f32_swiglu_kE", expert="swiglu", E=4, k=4, T=33),
    wl("f32_relu_one_token", T=1),
]

BF16_CASES = [
    wl("bf16_swiglu_ragged", T=1000, d=512, E=8, ffn=640, k=2, dtype="bf16", expert="swiglu"),
    wl("bf16_gelu_ragged", T=600, d=320, E=8, ffn=576, k=2, dtype="bf16", expert="gelu"),
    wl("bf16_relu", T=300, d=256, E=8, ffn=256, k=3, dtype="bf16", expert="relu"),
    wl("bf16_swiglu_sigmoid_groups", T=700, d=384, E=16, ffn=192, k=3, n_groups=4, topk_groups=2,
       dtype="bf16", expert="swiglu", score="sigmoid"),
    wl("bf16_swiglu_k1", T=257, d=128, E=8, ffn=128, k=1, dtype="bf16", expert="swiglu"),
    wl("bf16_swiglu_tall", T=1500, d=192, E=8, ffn=320, k=4, dtype="bf16", expert="swiglu"),
    # the router weight gradient split over 26 token chunks of 160 rows, the last one 100 rows
    wl("bf16_swiglu_router_split", T=4100, d=128, E=8, ffn=128, k=2, dtype="bf16", expert="swiglu"),
]


# router variants: correction bias (selection only), top-2-sum group score, route scale
VARIANT_CASES = [
    wl("f32_swiglu_bias_top2_scale", expert="swiglu", score="sigmoid", n_groups=4, topk_groups=2,
       e_bias=0.1, group_score="top2", route_scale=2.5),
    wl("f32_relu_softmax_top2_half", n_groups=2, topk_groups=1, group_score="top2", route_scale=0.5),
    wl("bf16_swiglu_bias_top2_scale", T=700, d=384, E=16, ffn=192, k=3, n_groups=4, topk_groups=2,
       dtype="bf16", expert="swiglu", score="sigmoid", e_bias=0.1, group_score="top2", route_scale=2.5),
    wl("bf16_gelu_bias_max", T=500, d=256, E=16, ffn=320, k=2, n_groups=4, topk_groups=2,
       dtype="bf16", expert="gelu", score="sigmoid", e_bias=0.2),
]


# shared-experts branch (one SwiGLU of hidden n_shared * ffn over every token)
SHARED_CASES = [
    wl("f32_swiglu_shared2", expert="swiglu", n_shared=2),
    wl("f32_relu_shared1", n_shared=1, T=33),
    wl("bf16_swiglu_shared_ragged", T=1000, d=512, E=8, ffn=640, k=2, dtype="bf16", expert="swiglu",
       n_shared=1),
    wl("bf16_gelu_shared2", T=600, d=320, E=8, ffn=576, k=2, dtype="bf16", expert="gelu", n_shared=2),
    wl("bf16_swiglu_sigmoid_groups_shared", T=700, d=384, E=16, ffn=192, k=3, n_groups=4, topk_groups=2,
       dtype="bf16", expert="swiglu", score="sigmoid", n_shared=3),
]


# the limits: k = MOE_MAX_K = 16 (the dispatch kernels' generic-k path), E = MOE_MAX_EXPERTS = 256
# with most experts below one 64-row tile (narrow tail tiles, some experts empty), and the
# compiled k = 6 specialisation of the dispatch kernels
LIMIT_CASES = [
    wl("f32_relu_k16_e16", E=16, k=16),
    wl("bf16_swiglu_k16", T=300, d=128, E=32, ffn=192, k=16, dtype="bf16", expert="swiglu"),
    wl("bf16_swiglu_e256_groups", T=512, d=128, E=256, ffn=128, k=8, n_groups=8, topk_groups=4,
       dtype="bf16", expert="swiglu", score="sigmoid"),
    wl("bf16_gelu_k6_groups", T=300, d=192, E=16, ffn=256, k=6, n_groups=8, topk_groups=4,
       dtype="bf16", expert="gelu", score="sigmoid"),
    # k = 8: the router dX contraction with the scatter in its epilogue, over a ragged last row
    # tile and column tile, with and without the shared branch's part
    wl("bf16_swiglu_k8_shared_ragged", T=700, d=320, E=16, ffn=192, k=8, dtype="bf16", expert="swiglu",
       n_shared=1),
    wl("bf16_gelu_k8_ragged", T=333, d=192, E=16, ffn=256, k=8, dtype="bf16", expert="gelu"),
    # router logits split over K into segments of 320, 320 and 192 columns (a ragged last one)
    wl("bf16_swiglu_router_ragged_split", T=300, d=832, E=8, ffn=128, k=2, dtype="bf16",
       expert="swiglu"),
]


def _inputs(w, seed=0):
    return W.make_inputs(w, seed=seed, masters=True)


@pytest.mark.parametrize("w", F32_CASES + BF16_CASES + VARIANT_CASES + SHARED_CASES + LIMIT_CASES,
                         ids=lambda w: w.name)
def test_forward_backward_parity(w):
    say(f"layer parity {w}")
    inp = _inputs(w)
    dY = W.make_upstream_grad(w)
    full_parity(w, inp, dY, aux_coef=0.3, label=w.name)


def test_empty_experts_get_zero_gradients():
    # gate rows 4..7 copy row 3: experts 5, 6, 7 can never win a tie against 3, 4 (k = 2)
    w = wl("bf16_empty", T=512, d=256, E=8, ffn=256, k=2, dtype="bf16", expert="swiglu")
    inp = _inputs(w)
    g = inp["Wg"].clone()
    g[4:] = g[3]
    inp["Wg"] = g
    inp["Wg_w"] = g.to(torch.bfloat16)
    run, fw, gr, _ = full_parity(w, inp, W.make_upstream_grad(w), aux_coef=0.1, label="empty")
    counts = run.routing["counts"].cpu().numpy()
    assert counts[5] == counts[6] == counts[7] == 0
    for n in ("dW1", "dW2", "dW3"):
        assert torch.count_nonzero(run.grads[n][5:]).item() == 0


def test_no_tokens():
    w = wl("f32_no_tokens", T=0)
    inp = _inputs(w)
    run = LayerRun(w, inp)
    run.forward()
    run.backward(torch.empty(0, w.d, device="cuda"), 0.5)
    torch.cuda.synchronize()
    assert run.routing["counts"].cpu().tolist() == [0] * w.E
    assert run.routing["offsets"].cpu().tolist() == [0] * (w.E + 1)
    assert float(run.routing["aux"][0]) == 0.0
    for n in ("dWg", "dW1", "dW2", "db1", "db2"):
        assert torch.count_nonzero(run.grads[n]).item() == 0, n


@pytest.mark.parametrize("w", [F32_CASES[2], BF16_CASES[0], BF16_CASES[3]], ids=lambda w: w.name)
def test_bitwise_deterministic(w):
    inp = _inputs(w)
    dY = W.make_upstream_grad(w).cuda()
    outs = []
    for _ in range(2):
        run = LayerRun(w, inp)
        run.forward()
        run.backward(dY, 0.2)
        torch.cuda.synchronize()
        outs.append({**{n: v.cpu() for n, v in run.routing.items()}, "Y": run.Y.cpu(),
                     **{n: v.cpu() for n, v in run.grads.items()}})
    for n in outs[0]:
        assert torch.equal(outs[0][n], outs[1][n]), n


def test_inputs_unchanged_and_calls_repeatable():
    w = BF16_CASES[0]
    inp = _inputs(w)
    run = LayerRun(w, inp)
    before = {n: v.clone() for n, v in run.weights.items() if v is not None}
    X0 = run.X.clone()
    dY = W.make_upstream_grad(w).cuda()
    dY0 = dY.clone()
    run.forward(); run.backward(dY, 0.2)
    Y1 = run.Y.clone(); g1 = {n: v.clone() for n, v in run.grads.items()}
    run.forward(); run.backward(dY, 0.2)
    torch.cuda.synchronize()
    assert torch.equal(run.X, X0) and torch.equal(dY, dY0)
    for n, v in before.items():
        assert torch.equal(run.weights[n], v), n
    assert torch.equal(run.Y, Y1)
    for n in g1:
        assert torch.equal(run.grads[n], g1[n]), n


EXPERT_GRADS = ("dW1", "dW2", "dW3", "dWs1", "dWs2", "dWs3")
PARAM_NAMES = ("Wg", "W1", "b1", "W2", "b2", "W3", "Ws1", "Ws3", "Ws2")


def train_step_parity(w, inp, label, fused=False):
    """moe_train_step against the oracle's forward, loss, backward and SGD.
    fused: the expert weight gradients are not passed, so the weight-gradient
    contractions apply the SGD step to W1, W2 (W3) themselves."""
    dev = "cuda"
    cfg = L.config(w)
    ws = L.alloc_workspace(cfg, dev)
    r = L.alloc_routing(w, dev)
    g = L.alloc_grads(w, dev)
    if fused:
        for n in EXPERT_GRADS:
            g.pop(n, None)
    Y = torch.empty(w.T, w.d, dtype=w.torch_dtype, device=dev)
    loss = torch.empty(3, dtype=torch.float32, device=dev)
    params = {}
    for n in PARAM_NAMES:
        if inp.get(n) is not None:
            params[n] = inp[n].clone().to(dev)
            params[n + "_w"] = inp[n + "_w"].clone().to(dev)
    if inp.get("e_bias") is not None:
        params["e_bias"] = inp["e_bias"].to(dev)
    X, Yt = inp["X"].to(dev), inp["Yt"].to(dev)
    L.moe_train_step(cfg, X, Yt, params, w.lr, w.aux_coef, Y, r, g, loss, ws)
    torch.cuda.synchronize()
    rtol, atol = TOL[w.dtype]
    X64 = to64(inp["X"])
    P = oracle_params(inp)
    l64 = X64 @ P["Wg"].T
    resolved, _, _ = check_routing(r, l64, w, P["e_bias"], label)
    st = O.train_step(X64, to64(inp["Yt"]), P, shape_of(w), w.lr, w.aux_coef, topk_idx=resolved)
    say(f"[{label}] loss gpu {loss.tolist()} oracle {[st['mse'], st['fw']['aux'], st['loss']]}")
    assert_close("loss", to64(loss), [st["mse"], st["fw"]["aux"], st["loss"]], rtol, atol)
    assert_close("Y", to64(Y), st["fw"]["Y"], rtol, atol)
    for n in g:
        assert_close(n, to64(g[n]), st["grads"][n], rtol, atol)
    if "e_bias" in params:
        assert torch.equal(params["e_bias"].cpu(), inp["e_bias"]), "the correction bias was written"
    for n in PARAM_NAMES:
        if n not in params:
            continue
        new = to64(params[n])
        old = to64(inp[n])
        ulp = np.abs(np.spacing(new.astype(np.float32))).astype(np.float64)
        # the update itself, with one float32 ulp of the stored master allowed
        assert_close("update " + n, new - old, -w.lr * st["grads"]["d" + n], rtol, atol, extra_abs=ulp)
        if w.dtype == "bf16":
            assert torch.equal(params[n + "_w"].cpu(), params[n].cpu().to(torch.bfloat16)), n
        elif params[n + "_w"].data_ptr() != params[n].data_ptr():
            assert torch.equal(params[n + "_w"].cpu(), params[n].cpu()), n
    return params, loss


@pytest.mark.parametrize("w", [F32_CASES[0], F32_CASES[2], BF16_CASES[1], BF16_CASES[3],
                               VARIANT_CASES[0], VARIANT_CASES[2]], ids=lambda w: w.name)
def test_train_step_parity(w):
    train_step_parity(w, _inputs(w), w.name)


# skewed routing (Zipf gate rows, a tie block that leaves experts empty): the persistent
# weight gradients hand out segments of very different lengths, the longest first
SKEWED_PERSISTENT = wl("bf16_swiglu_skewed_queue", T=3000, d=256, E=32, ffn=320, k=4, dtype="bf16",
                       expert="swiglu", gate="zipf_tie")

FUSED_CASES = [F32_CASES[0], F32_CASES[2], BF16_CASES[0], BF16_CASES[1], BF16_CASES[2], BF16_CASES[5],
               VARIANT_CASES[2], SHARED_CASES[0], SHARED_CASES[2], SHARED_CASES[3], LIMIT_CASES[2],
               SKEWED_PERSISTENT, SKEWED_PERSISTENT.replace(name="bf16_swiglu_skewed_queue_fd",
                                                            fused_dispatch=1)]


@pytest.mark.parametrize("w", [SHARED_CASES[1], SHARED_CASES[4]], ids=lambda w: w.name)
def test_train_step_parity_shared(w):
    train_step_parity(w, _inputs(w), w.name)


@pytest.mark.parametrize("w", FUSED_CASES, ids=lambda w: w.name)
def test_train_step_fused_sgd_parity(w):
    train_step_parity(w, _inputs(w), w.name + "/fused", fused=True)


def _one_step(w, inp, fused, Wg_override=None):
    dev = "cuda"
    cfg = L.config(w)
    ws = L.alloc_workspace(cfg, dev)
    r = L.alloc_routing(w, dev)
    g = L.alloc_grads(w, dev)
    if fused:
        for n in EXPERT_GRADS:
            g.pop(n, None)
    Y = torch.empty(w.T, w.d, dtype=w.torch_dtype, device=dev)
    loss = torch.empty(3, dtype=torch.float32, device=dev)
    params = {}
    for n in PARAM_NAMES:
        if inp.get(n) is not None:
            params[n] = inp[n].clone().to(dev)
            params[n + "_w"] = inp[n + "_w"].clone().to(dev)
    L.moe_train_step(cfg, inp["X"].to(dev), inp["Yt"].to(dev), params, w.lr, w.aux_coef, Y, r, g,
                     loss, ws)
    torch.cuda.synchronize()
    out = {"Y": Y.cpu(), "loss": loss.cpu(), **{n: v.cpu() for n, v in params.items()},
           **{"grad " + n: v.cpu() for n, v in g.items() if n not in EXPERT_GRADS},
           **{"routing " + n: v.cpu() for n, v in r.items()}}
    return out


@pytest.mark.parametrize("w", [F32_CASES[2], BF16_CASES[0], BF16_CASES[1], BF16_CASES[5], SHARED_CASES[0],
                               SHARED_CASES[2], LIMIT_CASES[2], SKEWED_PERSISTENT],
                         ids=lambda w: w.name)
def test_fused_sgd_equals_stored_gradient_step(w):
    """The fused step and the step through stored gradients give bitwise the same
    parameters, outputs and remaining gradients: the gradient is the same float32
    sum and each element takes the same fused multiply-add.  (In bf16 the fused
    step's weight gradients run persistent, from per-XCD-group tile queues, and the
    stored step's do not: equality also shows that every tile was handed out once.)"""
    inp = _inputs(w)
    a = _one_step(w, inp, fused=False)
    b = _one_step(w, inp, fused=True)
    assert a.keys() == b.keys()
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_fused_sgd_with_empty_experts():
    """Experts that receive no rows keep their weights (their gradient is zero) in the
    fused step too, and their working copies are rewritten from the masters."""
    w = wl("bf16_empty_fused", T=512, d=256, E=8, ffn=256, k=2, dtype="bf16", expert="swiglu")
    inp = _inputs(w)
    g = inp["Wg"].clone()
    g[4:] = g[3]
    inp["Wg"] = g
    inp["Wg_w"] = g.to(torch.bfloat16)
    out = _one_step(w, inp, fused=True)
    assert out["routing counts"][5:].tolist() == [0, 0, 0]
    for n in ("W1", "W2", "W3"):
        assert torch.equal(out[n][5:], inp[n][5:]), n
        assert torch.equal(out[n + "_w"][5:], inp[n][5:].to(torch.bfloat16)), n
    ref = _one_step(w, inp, fused=False)
    for n in ref:
        assert torch.equal(ref[n], out[n]), n


def test_train_step_rejects_partial_expert_gradients():
    """dW1, dW2 (dW3) are given together or not at all."""
    w = BF16_CASES[4]
    dev = "cuda"
    cfg = L.config(w)
    ws = L.alloc_workspace(cfg, dev)
    r = L.alloc_routing(w, dev)
    inp = _inputs(w)
    params = {}
    for n in ("Wg", "W1", "W2", "W3"):
        params[n] = inp[n].clone().to(dev)
        params[n + "_w"] = inp[n + "_w"].clone().to(dev)
    keep = {n: v.clone() for n, v in params.items()}
    Y = torch.empty(w.T, w.d, dtype=w.torch_dtype, device=dev)
    loss = torch.empty(3, dtype=torch.float32, device=dev)
    for drop in (("dW1",), ("dW3",), ("dW1", "dW2")):
        g = L.alloc_grads(w, dev)
        for n in drop:
            g.pop(n)
        with pytest.raises(L.MoeError) as ei:
            L.moe_train_step(cfg, inp["X"].to(dev), inp["Yt"].to(dev), params, w.lr, w.aux_coef, Y, r,
                             g, loss, ws)
        assert L.STATUS[ei.value.status] == "MOE_ERR_NULL_PTR"
    torch.cuda.synchronize()
    for n, v in keep.items():
        assert torch.equal(params[n], v), n


def test_train_step_rejects_partial_shared_gradients():
    """With a shared branch its gradients join the all-or-none rule."""
    w = SHARED_CASES[2]
    dev = "cuda"
    cfg = L.config(w)
    ws = L.alloc_workspace(cfg, dev)
    r = L.alloc_routing(w, dev)
    inp = _inputs(w)
    params = {}
    for n in PARAM_NAMES:
        if inp.get(n) is not None:
            params[n] = inp[n].clone().to(dev)
            params[n + "_w"] = inp[n + "_w"].clone().to(dev)
    keep = {n: v.clone() for n, v in params.items()}
    Y = torch.empty(w.T, w.d, dtype=w.torch_dtype, device=dev)
    loss = torch.empty(3, dtype=torch.float32, device=dev)
    for drop in (("dW1", "dW2", "dW3"), ("dWs2",), ("dWs1", "dWs2", "dWs3")):
        g = L.alloc_grads(w, dev)
        for n in drop:
            g.pop(n)
        with pytest.raises(L.MoeError) as ei:
            L.moe_train_step(cfg, inp["X"].to(dev), inp["Yt"].to(dev), params, w.lr, w.aux_coef, Y, r,
                             g, loss, ws)
        assert L.STATUS[ei.value.status] == "MOE_ERR_NULL_PTR"
    torch.cuda.synchronize()
    for n, v in keep.items():
        assert torch.equal(params[n], v), n


@pytest.mark.parametrize("w", [F32_CASES[0], BF16_CASES[3]], ids=lambda w: w.name)
def test_router_path_alone(w):
    """dY = 0: only the aux loss drives gradients, so dX is the router path dl Wg
    alone and every expert gradient is exactly zero."""
    inp = _inputs(w)
    dY = torch.zeros(w.T, w.d, dtype=w.torch_dtype)
    run, fw, gr, _ = full_parity(w, inp, dY, aux_coef=0.7, check_saved=False, label="router-only")
    for n in ("dW1", "dW2", "dW3", "db1", "db2"):
        if n in run.grads:
            assert torch.count_nonzero(run.grads[n]).item() == 0, n
    assert torch.count_nonzero(run.grads["dX"]).item() > 0


@pytest.mark.parametrize("fused", [False, True], ids=["stored", "fused"])
def test_train_step_no_tokens_bf16_shared(fused):
    """T = 0 through the bf16 path with a shared branch: every kernel runs on empty
    row segments, the loss is zero, the gradients are exact zeros and the step leaves
    every master as it was (its bf16 copy is the master rounded)."""
    w = wl("bf16_no_tokens_shared", T=0, d=128, E=8, ffn=128, k=2, dtype="bf16", expert="swiglu", n_shared=1)
    dev = "cuda"
    cfg = L.config(w)
    ws = L.alloc_workspace(cfg, dev)
    r = L.alloc_routing(w, dev)
    g = L.alloc_grads(w, dev)
    if fused:
        for n in EXPERT_GRADS:
            g.pop(n, None)
    inp = _inputs(w)
    params = {}
    for n in PARAM_NAMES:
        if inp.get(n) is not None:
            params[n] = inp[n].clone().to(dev)
            params[n + "_w"] = inp[n + "_w"].clone().to(dev)
    Y = torch.empty(0, w.d, dtype=w.torch_dtype, device=dev)
    loss = torch.full((3,), 7.0, dtype=torch.float32, device=dev)
    L.moe_train_step(cfg, inp["X"].to(dev), inp["Yt"].to(dev), params, w.lr, w.aux_coef, Y, r, g, loss, ws)
    torch.cuda.synchronize()
    assert loss.tolist() == [0.0, 0.0, 0.0]
    assert r["counts"].cpu().tolist() == [0] * w.E
    for n, v in g.items():
        assert torch.count_nonzero(v).item() == 0, n
    for n in PARAM_NAMES:
        if n in params:
            assert torch.equal(params[n].cpu(), inp[n]), n
            assert torch.equal(params[n + "_w"].cpu(), inp[n].to(torch.bfloat16)), n
