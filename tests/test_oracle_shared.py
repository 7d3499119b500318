"""Pins of the oracle's shared-experts branch (reading R20): one SwiGLU over
every token, added to the routed combine with no gate.

The branch is pinned by reduction to the single routed expert (itself pinned
against scalar loops in test_oracle_layer.py), by central differences of the
loss, by a torch float64 autograd cross-check of a dense formulation, and by
closed forms (zero output projection, linearity in Ws2, the SGD update).
"""
import math

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests.test_oracle_layer import _rand_params


def _shared(rng, d, hs):
    return {"Ws1": rng.normal(size=(hs, d)) / math.sqrt(d),
            "Ws3": rng.normal(size=(hs, d)) / math.sqrt(d),
            "Ws2": rng.normal(size=(d, hs)) / math.sqrt(hs)}


def _layer(rng, T, d, ffn, E, k, expert, hs, score="softmax"):
    X = rng.normal(size=(T, d))
    Yt = rng.normal(size=(T, d))
    P = _rand_params(rng, E, d, ffn, expert)
    P.update(_shared(rng, d, hs))
    return X, Yt, P, O.Shape(E=E, k=k, score=score, expert=expert)


@pytest.mark.parametrize("expert", ["gelu", "swiglu"])
def test_shared_branch_is_one_routed_expert_over_every_token(expert):
    """Y with the branch minus Y without it equals a routed layer with one SwiGLU
    expert, k = 1 (gate 1) and the shared weights; so do the branch's weight
    gradients and its part of dX."""
    rng = np.random.default_rng(21)
    T, d, ffn, E, k, hs = 11, 6, 5, 4, 2, 7
    X, Yt, P, shp = _layer(rng, T, d, ffn, E, k, expert, hs)
    base = {n: v for n, v in P.items() if not n.startswith("Ws")}
    fw = O.layer_forward(X, P, shp)
    fw0 = O.layer_forward(X, base, shp)
    one = {"Wg": np.zeros((1, d)), "W1": P["Ws1"][None], "W3": P["Ws3"][None], "W2": P["Ws2"][None],
           "b1": None, "b2": None}
    shp1 = O.Shape(E=1, k=1, expert="swiglu")
    fw1 = O.layer_forward(X, one, shp1)
    assert np.allclose(fw["Y"] - fw0["Y"], fw1["Y"], rtol=1e-12, atol=1e-13)
    assert np.array_equal(fw["topk_idx"], fw0["topk_idx"])
    dY = rng.normal(size=(T, d))
    g = O.layer_backward(X, P, shp, fw, dY, aux_coef=0.2)
    g0 = O.layer_backward(X, base, shp, fw0, dY, aux_coef=0.2)
    g1 = O.layer_backward(X, one, shp1, fw1, dY, aux_coef=0.0)
    for a, b in (("dWs1", "dW1"), ("dWs2", "dW2"), ("dWs3", "dW3")):
        assert np.allclose(g[a], g1[b][0], rtol=1e-12, atol=1e-13), a
    assert np.allclose(g["dX"] - g0["dX"], g1["dX"], rtol=1e-11, atol=1e-13)
    for n in ("dWg", "dW1", "dW2", "dW3", "db1", "db2"):       # the routed part does not move
        if n in g0:
            assert np.array_equal(g[n], g0[n]), n


def _loss(X, Yt, P, shp, aux_coef, idx_ref):
    fw = O.layer_forward(X, P, shp)
    assert np.array_equal(fw["topk_idx"], idx_ref), "routing flipped under the perturbation"
    m, _ = O.mse(fw["Y"], Yt)
    return m + aux_coef * fw["aux"]


@pytest.mark.parametrize("expert", ["relu", "swiglu"])
def test_shared_central_differences(expert):
    rng = np.random.default_rng(22)
    T, d, ffn, E, k, hs = 8, 4, 3, 4, 2, 5
    X, Yt, P, shp = _layer(rng, T, d, ffn, E, k, expert, hs, score="sigmoid")
    if expert == "relu":                      # keep pre-activations off the kink
        for e in range(E):
            assert np.all(np.abs(X @ P["W1"][e].T + P["b1"][e]) > 1e-4)
    aux_coef = 0.3
    st = O.train_step(X, Yt, P, shp, lr=0.0, aux_coef=aux_coef)
    idx = st["fw"]["topk_idx"]
    for name in ("Ws1", "Ws2", "Ws3", "X"):
        theta = X if name == "X" else P[name]
        ref = st["grads"]["dX" if name == "X" else "d" + name]
        num = np.zeros_like(theta)
        for j in np.ndindex(theta.shape):
            old = theta[j]
            h = 1e-6 * max(1.0, abs(old))
            theta[j] = old + h
            lp = _loss(X, Yt, P, shp, aux_coef, idx)
            theta[j] = old - h
            lm = _loss(X, Yt, P, shp, aux_coef, idx)
            theta[j] = old
            num[j] = (lp - lm) / (2 * h)
        err = np.abs(num - ref).max() / max(1e-12, np.abs(ref).max())
        assert err < 1e-6, (name, err)


def test_shared_against_torch_autograd():
    rng = np.random.default_rng(23)
    T, d, ffn, E, k, hs = 20, 8, 6, 8, 3, 10
    X, Yt, P, _ = _layer(rng, T, d, ffn, E, k, "swiglu", hs)
    shp = O.Shape(E=E, k=k, n_groups=4, topk_groups=2, score="sigmoid", expert="swiglu")
    st = O.train_step(X, Yt, P, shp, lr=0.0, aux_coef=0.05)
    idx = st["fw"]["topk_idx"]
    t = {n: torch.tensor(v, requires_grad=True) for n, v in P.items() if v is not None}
    tX = torch.tensor(X, requires_grad=True)
    logits = tX @ t["Wg"].T
    prob = torch.sigmoid(logits)
    mask = torch.zeros(T, E, dtype=torch.float64)
    mask.scatter_(1, torch.as_tensor(idx), 1.0)
    G = prob * mask / (prob * mask).sum(1, keepdim=True)
    Y = torch.zeros(T, d, dtype=torch.float64)
    for e in range(E):
        a = torch.nn.functional.silu(tX @ t["W1"][e].T) * (tX @ t["W3"][e].T)
        Y = Y + G[:, e:e + 1] * (a @ t["W2"][e].T)
    Y = Y + (torch.nn.functional.silu(tX @ t["Ws1"].T) * (tX @ t["Ws3"].T)) @ t["Ws2"].T
    q = prob / prob.sum(1, keepdim=True)
    aux = E * (mask.sum(0) / (T * k) * q.mean(0)).sum()
    loss = ((Y - torch.tensor(Yt)) ** 2).mean() + 0.05 * aux
    loss.backward()
    assert np.allclose(Y.detach().numpy(), st["fw"]["Y"], rtol=1e-12, atol=1e-13)
    for n in ("Ws1", "Ws2", "Ws3", "W1", "W2", "W3", "Wg"):
        assert np.allclose(t[n].grad.numpy(), st["grads"]["d" + n], rtol=1e-10, atol=1e-13), n
    assert np.allclose(tX.grad.numpy(), st["grads"]["dX"], rtol=1e-10, atol=1e-13)


def test_zero_output_projection_and_linearity():
    rng = np.random.default_rng(24)
    T, d, ffn, E, k, hs = 9, 5, 4, 4, 2, 6
    X, Yt, P, shp = _layer(rng, T, d, ffn, E, k, "swiglu", hs)
    base = {n: v for n, v in P.items() if not n.startswith("Ws")}
    dY = rng.normal(size=(T, d))
    z = dict(P, Ws2=np.zeros_like(P["Ws2"]))
    fz, f0 = O.layer_forward(X, z, shp), O.layer_forward(X, base, shp)
    assert np.array_equal(fz["Y"], f0["Y"])
    gz = O.layer_backward(X, z, shp, fz, dY, 0.1)
    g0 = O.layer_backward(X, base, shp, f0, dY, 0.1)
    assert not gz["dWs1"].any() and not gz["dWs3"].any()     # no path to the loss
    assert np.array_equal(gz["dX"], g0["dX"])
    # dWs2 = dY^T A with A = silu(X Ws1^T) * (X Ws3^T), which does not depend on Ws2
    A = fz["shared"]["A"]
    assert np.allclose(gz["dWs2"], dY.T @ A, rtol=1e-13, atol=1e-14)
    # the branch is linear in Ws2
    f1 = O.layer_forward(X, P, shp)
    f3 = O.layer_forward(X, dict(P, Ws2=3.0 * P["Ws2"]), shp)
    assert np.allclose(f3["Y"] - f0["Y"], 3.0 * (f1["Y"] - f0["Y"]), rtol=1e-12, atol=1e-13)


def test_shared_weights_take_the_sgd_step():
    rng = np.random.default_rng(25)
    X, Yt, P, shp = _layer(rng, 7, 4, 3, 4, 2, "swiglu", 5)
    st = O.train_step(X, Yt, P, shp, lr=0.25, aux_coef=0.1)
    for n in ("Ws1", "Ws2", "Ws3"):
        assert np.allclose(st["params"][n], P[n] - 0.25 * st["grads"]["d" + n], rtol=0, atol=1e-15), n
