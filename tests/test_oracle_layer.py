"""Pins of the oracle's layer forward, backward and SGD.

* a hand-worked example with exact fractions (tests/golden/hand_worked_relu.json)
* E = 1, k = 1 reduces the layer to a dense MLP / SwiGLU written out here
* identical experts: the gate path gives the router no gradient
* central differences of every parameter and input gradient (float64)
* an independent dense formulation differentiated by torch autograd (CPU)
* closed forms of the activations and the optimiser step
* metamorphic checks: token permutation and expert relabelling
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _val(s):
    s = s.strip()
    neg = s.startswith("-")
    s = s.lstrip("-")
    if s.startswith("ln"):
        v = math.log(float(s[2:]))
    else:
        v = float(Fraction(s))
    return -v if neg else v


def _arr(x):
    if isinstance(x, str):
        return _val(x)
    return np.array([_arr(v) for v in x], dtype=np.float64)


def test_hand_worked_golden():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_relu.json")))
    inp, exp = g["inputs"], g["expected"]
    P = {n: _arr(inp[n]) for n in ("Wg", "W1", "b1", "W2", "b2")}
    P["W3"] = None
    X, Yt = _arr(inp["X"]), _arr(inp["Yt"])
    shp = O.Shape(E=3, k=2, score="softmax", expert="relu")
    st = O.train_step(X, Yt, P, shp, lr=0.0, aux_coef=0.01)
    fw, gr = st["fw"], st["grads"]
    r = fw["routing"]
    assert fw["topk_idx"].tolist() == exp["topk_idx"]
    assert r.counts.tolist() == exp["counts"]
    assert r.offsets.tolist() == exp["offsets"]
    assert r.slot_of.tolist() == exp["slot_of"]
    assert r.token_of.tolist() == exp["token_of"]
    tol = dict(rtol=1e-14, atol=1e-15)
    assert np.allclose(fw["gates"], _arr(exp["gates"]), **tol)
    assert np.allclose(O.scores(fw["logits"], "softmax"), _arr(exp["probs"]), **tol)
    assert np.allclose(fw["Y"], _arr(exp["Y"]), **tol)
    assert abs(fw["aux"] - _val(exp["aux"])) < 1e-14
    assert abs(st["mse"] - _val(exp["mse"])) < 1e-15
    assert np.allclose(gr["dgate"], _arr(exp["dgate"]), **tol)
    assert np.allclose(gr["db2"], _arr(exp["db2"]), **tol)
    assert np.all(gr["dW1"][2] == 0) and np.all(gr["dW2"][2] == 0) and np.all(gr["db1"][2] == 0)


def _rand_params(rng, E, d, ffn, expert, bias_scale=0.3):
    P = {"Wg": rng.normal(size=(E, d)),
         "W1": rng.normal(size=(E, ffn, d)) / math.sqrt(d),
         "W2": rng.normal(size=(E, d, ffn)) / math.sqrt(ffn),
         "W3": rng.normal(size=(E, ffn, d)) / math.sqrt(d) if expert == "swiglu" else None}
    if expert != "swiglu":
        P["b1"] = rng.normal(size=(E, ffn)) * bias_scale
        P["b2"] = rng.normal(size=(E, d)) * bias_scale
    else:
        P["b1"] = P["b2"] = None
    return P


@pytest.mark.parametrize("expert", ["relu", "gelu", "swiglu"])
def test_single_expert_is_dense_layer(expert):
    rng = np.random.default_rng(5)
    T, d, ffn = 9, 6, 10
    X = rng.normal(size=(T, d))
    Yt = rng.normal(size=(T, d))
    P = _rand_params(rng, 1, d, ffn, expert)
    shp = O.Shape(E=1, k=1, expert=expert)
    st = O.train_step(X, Yt, P, shp, lr=0.1, aux_coef=0.5)
    W1, W2 = P["W1"][0], P["W2"][0]
    # dense forward written out with scalar math per element
    Y = np.zeros((T, d))
    for t in range(T):
        if expert == "swiglu":
            W3 = P["W3"][0]
            a = []
            for j in range(ffn):
                h1 = sum(W1[j, c] * X[t, c] for c in range(d))
                h3 = sum(W3[j, c] * X[t, c] for c in range(d))
                a.append(h1 / (1 + math.exp(-h1)) * h3)
            for c in range(d):
                Y[t, c] = sum(W2[c, j] * a[j] for j in range(ffn))
        else:
            a = []
            for j in range(ffn):
                h = sum(W1[j, c] * X[t, c] for c in range(d)) + P["b1"][0, j]
                a.append(max(h, 0.0) if expert == "relu" else 0.5 * h * (1 + math.erf(h / math.sqrt(2))))
            for c in range(d):
                Y[t, c] = sum(W2[c, j] * a[j] for j in range(ffn)) + P["b2"][0, c]
    assert np.allclose(st["fw"]["Y"], Y, rtol=1e-12, atol=1e-13)
    assert abs(st["fw"]["aux"] - 1.0) < 1e-15        # one expert takes everything
    assert np.all(st["grads"]["dWg"] == 0.0)        # softmax over one expert is constant
    assert abs(st["mse"] - ((Y - Yt) ** 2).mean()) < 1e-13


def test_identical_experts_give_router_no_gate_gradient():
    rng = np.random.default_rng(6)
    T, d, ffn, E = 12, 5, 7, 4
    X = rng.normal(size=(T, d))
    P = _rand_params(rng, 1, d, ffn, "gelu")
    for n in ("W1", "W2", "b1", "b2"):
        P[n] = np.repeat(P[n], E, axis=0)
    P["Wg"] = rng.normal(size=(E, d))
    for score in ("softmax", "sigmoid"):
        shp = O.Shape(E=E, k=2, score=score, expert="gelu")
        fw = O.layer_forward(X, P, shp)
        dY = rng.normal(size=(T, d))
        g0 = O.layer_backward(X, P, shp, fw, dY, aux_coef=0.0)
        assert np.abs(g0["dWg"]).max() < 1e-13
        g1 = O.layer_backward(X, P, shp, fw, dY, aux_coef=0.3)
        assert np.abs(g1["dWg"]).max() > 1e-6


def _loss_fn(X, Yt, P, shp, aux_coef, idx_ref):
    fw = O.layer_forward(X, P, shp)
    assert np.array_equal(fw["topk_idx"], idx_ref), "routing flipped under the perturbation"
    m, _ = O.mse(fw["Y"], Yt)
    return m + aux_coef * fw["aux"]


def _tiny_problem(expert, score, G, seed):
    rng = np.random.default_rng(seed)
    T, d, ffn, E, k = 10, 4, 5, 4, 2
    for _ in range(200):
        X = rng.normal(size=(T, d))
        P = _rand_params(rng, E, d, ffn, expert, bias_scale=0.5)
        P["Wg"] = P["Wg"] * 1.5
        l = X @ P["Wg"].T
        srt = -np.sort(-l, axis=1)
        ok = np.all(np.abs(np.diff(srt, axis=1)) > 1e-3)
        if G > 1:
            gmax = l.reshape(T, G, E // G).max(2)
            ok &= np.all(np.abs(np.diff(-np.sort(-gmax, 1), axis=1)) > 1e-3)
        if expert == "relu":
            for e in range(E):
                ok &= np.all(np.abs(X @ P["W1"][e].T + P["b1"][e]) > 1e-3)
        if ok:
            return X, rng.normal(size=(T, d)), P, O.Shape(E=E, k=k, n_groups=G, topk_groups=1 if G > 1 else 1,
                                                          score=score, expert=expert)
    raise RuntimeError("no well-separated draw")


@pytest.mark.parametrize("expert", ["relu", "gelu", "swiglu"])
@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("G", [1, 2])
def test_central_differences(expert, score, G):
    X, Yt, P, shp = _tiny_problem(expert, score, G, seed=["relu", "gelu", "swiglu"].index(expert) * 10 + ["softmax", "sigmoid"].index(score) * 3 + G)
    if G > 1:
        shp = O.Shape(E=4, k=2, n_groups=2, topk_groups=1, score=score, expert=expert)
    aux_coef = 0.37
    st = O.train_step(X, Yt, P, shp, lr=0.0, aux_coef=aux_coef)
    idx = st["fw"]["topk_idx"]
    grads = st["grads"]
    checks = [(n, "d" + n) for n in ("Wg", "W1", "b1", "W2", "b2", "W3") if P.get(n) is not None]
    for name, gname in checks:
        theta = P[name]
        num = np.zeros_like(theta)
        for j in np.ndindex(theta.shape):
            h = 1e-6 * max(1.0, abs(theta[j]))
            old = theta[j]
            theta[j] = old + h
            lp = _loss_fn(X, Yt, P, shp, aux_coef, idx)
            theta[j] = old - h
            lm = _loss_fn(X, Yt, P, shp, aux_coef, idx)
            theta[j] = old
            num[j] = (lp - lm) / (2 * h)
        err = np.abs(num - grads[gname]).max() / max(1e-12, np.abs(grads[gname]).max())
        assert err < 1e-6, (name, err)
    num = np.zeros_like(X)
    for j in np.ndindex(X.shape):
        old = X[j]
        h = 1e-6 * max(1.0, abs(old))
        X[j] = old + h
        lp = _loss_fn(X, Yt, P, shp, aux_coef, idx)
        X[j] = old - h
        lm = _loss_fn(X, Yt, P, shp, aux_coef, idx)
        X[j] = old
        num[j] = (lp - lm) / (2 * h)
    err = np.abs(num - grads["dX"]).max() / np.abs(grads["dX"]).max()
    assert err < 1e-6, ("X", err)


def _torch_dense_loss(X, Yt, P, shp, idx, aux_coef):
    """Dense formulation: every expert on every token, weighted by a sparse gate matrix."""
    T, d = X.shape
    E = shp.E
    logits = X @ P["Wg"].T
    if shp.score == "softmax":
        prob = torch.softmax(logits, dim=1)
        q = prob
    else:
        prob = torch.sigmoid(logits)
        q = prob / prob.sum(1, keepdim=True)
    mask = torch.zeros(T, E, dtype=torch.float64)
    mask.scatter_(1, torch.as_tensor(idx), 1.0)
    wsel = prob * mask
    G = wsel / wsel.sum(1, keepdim=True)
    Y = torch.zeros(T, d, dtype=torch.float64)
    for e in range(E):
        if shp.expert == "swiglu":
            a = torch.nn.functional.silu(X @ P["W1"][e].T) * (X @ P["W3"][e].T)
            out = a @ P["W2"][e].T
        else:
            h = X @ P["W1"][e].T + P["b1"][e]
            a = torch.relu(h) if shp.expert == "relu" else torch.nn.functional.gelu(h)
            out = a @ P["W2"][e].T + P["b2"][e]
        Y = Y + G[:, e:e + 1] * out
    f = mask.sum(0) / (T * shp.k)
    aux = E * (f * q.mean(0)).sum()
    return ((Y - Yt) ** 2).mean() + aux_coef * aux, Y


@pytest.mark.parametrize("expert", ["relu", "gelu", "swiglu"])
@pytest.mark.parametrize("score,G,TG", [("softmax", 1, 1), ("sigmoid", 4, 2)])
def test_against_torch_autograd_dense_formulation(expert, score, G, TG):
    rng = np.random.default_rng(11)
    T, d, ffn, E, k = 24, 8, 12, 8, 3
    X = rng.normal(size=(T, d))
    Yt = rng.normal(size=(T, d))
    P = _rand_params(rng, E, d, ffn, expert)
    shp = O.Shape(E=E, k=k, n_groups=G, topk_groups=TG, score=score, expert=expert)
    st = O.train_step(X, Yt, P, shp, lr=0.0, aux_coef=0.05)
    tP = {n: (None if v is None else torch.tensor(v, requires_grad=True)) for n, v in P.items()}
    tX = torch.tensor(X, requires_grad=True)
    loss, Y = _torch_dense_loss(tX, torch.tensor(Yt), tP, shp, st["fw"]["topk_idx"], 0.05)
    loss.backward()
    assert np.allclose(Y.detach().numpy(), st["fw"]["Y"], rtol=1e-12, atol=1e-13)
    assert abs(loss.item() - st["loss"]) < 1e-13
    for n in ("Wg", "W1", "b1", "W2", "b2", "W3"):
        if P.get(n) is None:
            continue
        assert np.allclose(tP[n].grad.numpy(), st["grads"]["d" + n], rtol=1e-10, atol=1e-13), n
    assert np.allclose(tX.grad.numpy(), st["grads"]["dX"], rtol=1e-10, atol=1e-13)


def test_activation_closed_forms():
    xs = np.array([-3.0, -1.0, -1e-3, 0.0, 1e-3, 0.5, 2.0, 7.0])
    for x, gv, gg in zip(xs, O.gelu(xs), O.gelu_grad(xs)):
        phi = 0.5 * (1 + math.erf(x / math.sqrt(2)))
        assert abs(gv - x * phi) < 1e-15
        assert abs(gg - (phi + x * math.exp(-x * x / 2) / math.sqrt(2 * math.pi))) < 1e-15
    for x, sv, sg in zip(xs, O.silu(xs), O.silu_grad(xs)):
        s = 1 / (1 + math.exp(-x))
        assert abs(sv - x * s) < 1e-15
        h = 1e-6
        fd = ((x + h) / (1 + math.exp(-(x + h))) - (x - h) / (1 + math.exp(-(x - h)))) / (2 * h)
        assert abs(sg - fd) < 1e-8
    assert O.relu(np.array([-1.0, 0.0, 2.0])).tolist() == [0.0, 0.0, 2.0]
    assert O.relu_grad(np.array([-1.0, 0.0, 2.0])).tolist() == [0.0, 0.0, 1.0]
    # GELU(1) from the tabulated normal CDF value 0.8413447460685429
    assert abs(O.gelu(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15


def test_mse_and_sgd_closed_forms():
    Y = np.full((3, 4), 2.5)
    Yt = np.full((3, 4), 0.5)
    m, dY = O.mse(Y, Yt)
    assert m == 4.0 and np.all(dY == 2 * 2.0 / 12)
    th = np.array([1.0, -2.0])
    assert O.sgd(th, np.array([0.5, 0.25]), 0.1).tolist() == [1.0 - 0.05, -2.0 - 0.025]


def test_token_permutation_metamorphic():
    rng = np.random.default_rng(21)
    T, d, ffn, E = 16, 6, 8, 8
    X = rng.normal(size=(T, d))
    Yt = rng.normal(size=(T, d))
    P = _rand_params(rng, E, d, ffn, "swiglu")
    shp = O.Shape(E=E, k=3, n_groups=4, topk_groups=2, score="sigmoid", expert="swiglu")
    a = O.train_step(X, Yt, P, shp, lr=0.0, aux_coef=0.1)
    perm = rng.permutation(T)
    b = O.train_step(X[perm], Yt[perm], P, shp, lr=0.0, aux_coef=0.1)
    assert np.allclose(b["fw"]["Y"], a["fw"]["Y"][perm], rtol=1e-12, atol=1e-14)
    assert np.allclose(b["grads"]["dX"], a["grads"]["dX"][perm], rtol=1e-10, atol=1e-14)
    for n in ("dW1", "dW2", "dW3", "dWg"):
        assert np.allclose(b["grads"][n], a["grads"][n], rtol=1e-10, atol=1e-14)
    assert abs(a["fw"]["aux"] - b["fw"]["aux"]) < 1e-14
    assert np.array_equal(a["fw"]["routing"].counts, b["fw"]["routing"].counts)


def test_expert_relabel_metamorphic():
    rng = np.random.default_rng(22)
    T, d, ffn, E = 20, 6, 8, 6
    X = rng.normal(size=(T, d))
    P = _rand_params(rng, E, d, ffn, "gelu")
    shp = O.Shape(E=E, k=2, score="softmax", expert="gelu")
    a = O.layer_forward(X, P, shp)
    perm = rng.permutation(E)
    Q = {n: (None if v is None else v[perm]) for n, v in P.items()}
    b = O.layer_forward(X, Q, shp)
    assert np.allclose(a["Y"], b["Y"], rtol=1e-12, atol=1e-14)
    assert np.array_equal(perm[b["topk_idx"]], a["topk_idx"])


@pytest.mark.parametrize("expert,score,G,TG", [("swiglu", "sigmoid", 4, 2), ("relu", "softmax", 1, 1),
                                               ("gelu", "softmax", 2, 1)])
def test_streamed_step_equals_train_step(expert, score, G, TG):
    """The per-expert streamed step (used where the expert weights do not fit in host
    memory at once) gives train_step's loss, Y, dX, dWg and expert updates, with an
    expert left empty so that its zero gradients come out of the empty segment."""
    rng = np.random.default_rng(11)
    T, d, E, ffn, k = 40, 12, 8, 10, 2
    P = _rand_params(rng, E, d, ffn, expert)
    X = np.abs(rng.normal(size=(T, d)))
    P["Wg"][E - 1] = -10.0 * np.abs(P["Wg"][E - 1])   # far below every other logit: never picked
    Yt = rng.normal(size=(T, d))
    shp = O.Shape(E=E, k=k, n_groups=G, topk_groups=TG, score=score, expert=expert)
    ref = O.train_step(X, Yt, P, shp, lr=0.05, aux_coef=0.01)
    assert ref["fw"]["routing"].counts[E - 1] == 0

    def get(e):
        return {n: P[n][e] for n in ("W1", "W2", "W3", "b1", "b2") if P[n] is not None}

    keep = (0, 3, E - 1)
    st = O.train_step_streamed(X, Yt, P["Wg"], get, shp, lr=0.05, aux_coef=0.01, keep=keep)
    tol = dict(rtol=1e-12, atol=1e-14)
    assert np.array_equal(st["routing"].topk_idx, ref["fw"]["topk_idx"])
    for a, b in ((st["mse"], ref["mse"]), (st["aux"], ref["fw"]["aux"]), (st["loss"], ref["loss"])):
        assert abs(a - b) <= 1e-13 * max(1.0, abs(b))
    assert np.allclose(st["Y"], ref["fw"]["Y"], **tol)
    assert np.allclose(st["dY"], ref["dY"], **tol)
    assert np.allclose(st["dgate"], ref["grads"]["dgate"], **tol)
    assert np.allclose(st["dX"], ref["grads"]["dX"], **tol)
    assert np.allclose(st["dWg"], ref["grads"]["dWg"], **tol)
    for e in keep:
        for n, g in st["experts"][e]["grads"].items():
            assert np.allclose(g, ref["grads"][n][e], **tol), (e, n)
        for n, v in st["experts"][e]["params"].items():
            assert np.allclose(v, ref["params"][n][e], **tol), (e, n)
    assert all(np.all(g == 0) for g in st["experts"][E - 1]["grads"].values())
    # a caller-supplied dY replaces the MSE gradient in the backward
    dY = rng.normal(size=(T, d))
    sd = O.train_step_streamed(X, Yt, P["Wg"], get, shp, lr=0.05, aux_coef=0.01, keep=keep, dY=dY)
    gr = O.layer_backward(X, P, shp, ref["fw"], dY, 0.01)
    assert np.allclose(sd["dX"], gr["dX"], **tol)
    assert np.allclose(sd["dWg"], gr["dWg"], **tol)
    for e in keep:
        for n, g in sd["experts"][e]["grads"].items():
            assert np.allclose(g, gr[n][e], **tol), (e, n)
