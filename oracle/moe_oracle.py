"""Float64 CPU oracle of the trainable sparse mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it and
shares no code with it; the two meet only on seeded inputs.

Every function is the plain definition of one step, in float64, written for a
reader to check against the pages by eye:

  [Outline]  "Trainable MoE in CUDA" course outline (seven parts, each with a
             one-sentence statement of what the part computes).
  [Lesson29] "Define Expert Mlp Forward And Backward" (the expert MLP lesson,
             its "Prove it works" and "Common mistakes" lists).
  [Essay]    "Trainable MoE in CUDA" article, section "Make mathematical
             equivalence survive finite precision".
  [InfraLab] "AI Infra Kernel Lab" README, sections "Project status" and
             "Numerical contracts".

Where the pages leave a step open, the reading taken is named in the
docstring of the function that applies it (R1..R12 and R17..R20 below; the
numbers in between concern the workloads, i.e. how inputs are drawn, the
learning rates and the empty case, rather than a step of the layer).

  R1  group score = largest member logit (group-limited selection).
  R2  selection compares router logits (same order as the scores, since
      softmax and sigmoid are strictly increasing per token); key (-value, id)
      for experts and for groups, so ties go to the smaller id; output order is
      that key's order; +0.0 and -0.0 tie.
  R3  gates are always renormalised over the k selected experts.
  R4  aux = E * sum_e f_e * P_e, f_e = count_e / (T*k), P_e = mean_t q_te;
      q = softmax probabilities, or sigmoid scores normalised over the E
      experts; f carries no gradient.
  R5  MSE is the mean over all T*d elements.
  R6  GELU is the exact erf form.
  R7  rows of an expert segment are in ascending token order (stable).
  R8  dX is the full input gradient: expert path plus router path.
  R9  an expert with no rows gets exact-zero weight and bias gradients.
  R10 SGD: theta <- theta - lr * grad on float32 master copies; the working
      copy is the round-to-nearest-even bfloat16 of the new master.
  R11 the loss of every step is MSE + aux_coef * aux.
  R12 no intermediate rounding: inputs are taken at the exact values the
      caller holds (bfloat16 decoded exactly) and all arithmetic is float64.
  R17 correction bias (optional, sigmoid scoring only): it enters selection
      and nothing else.  Selection then ranks fp32 values v = fl32(s) + b
      (one fp32 addition of the correctly rounded sigmoid score and the fp32
      bias), the precision in which the kernel takes that integer decision;
      the gates and their gradients come from the unbiased scores.
  R18 top-2-sum group score (optional): a group's score is the sum of its two
      largest member values (fp32 when selection runs on fp32 values).  With
      this rule and no bias, selection ranks fl32(s).
  R19 route scale: the renormalised gates are multiplied by a constant
      (default 1); its gradient enters through the renormalisation.
  R20 shared experts (optional): a replicated branch that every token goes
      through, one SwiGLU with hidden size n_shared * ffn (weights Ws1, Ws3
      [Hs, d] and Ws2 [d, Hs]); its output is added to the routed combine with
      no gate, so its upstream gradient is dY itself; it is trained by the same
      SGD.

Parity pins (tests/test_oracle_*.py): brute-force top-k over all subsets,
gates summing to one and closed forms of the renormalisation, routing
conservation and the stable slot definition, aux == 1 under perfectly uniform
routing, the E=1/k=1 layer against a hand-written dense MLP, central
differences of every gradient, a torch float64 autograd cross-check,
closed-form activations, a hand-worked example under tests/golden/, and
metamorphic checks.  The group-score rule R1 and the aux formula R4 are pinned
only by internal consistency and the uniform-routing invariant, since the
pages print neither formula.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

# ----------------------------------------------------------------------------
# Part 1 building blocks: activations and their derivatives
# [Outline] Part 1 "CUDA Building Blocks": activations with backward passes.
# ----------------------------------------------------------------------------

_erf = np.vectorize(math.erf, otypes=[np.float64])


def relu(x):
    return np.maximum(x, 0.0)


def relu_grad(x):
    return (x > 0.0).astype(np.float64)


def gelu(x):
    """x * Phi(x), exact erf form (R6)."""
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def gelu_grad(x):
    """Phi(x) + x * phi(x)."""
    cdf = 0.5 * (1.0 + _erf(x / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
    return cdf + x * pdf


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    return x * sigmoid(x)


def silu_grad(x):
    s = sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


def softmax_rows(l):
    """Row-wise softmax with the row maximum subtracted ([Essay])."""
    m = l.max(axis=1, keepdims=True)
    z = np.exp(l - m)
    return z / z.sum(axis=1, keepdims=True)


ACT = {"relu": (relu, relu_grad), "gelu": (gelu, gelu_grad)}

# ----------------------------------------------------------------------------
# Part 3 router and Part 2 top-k gating utilities
# [Outline] Part 3 "Router": logits by a gate matmul, probabilities, top-k.
# [Outline] Part 2 "Top-K Gating Utilities": top-k per token, gates
#           normalised to a distribution, backward through the normalisation.
# [InfraLab] "Project status": group-limited selector, exact ties prefer the
#           smaller group/expert id; sigmoid scoring in the grouped gate.
# ----------------------------------------------------------------------------


def router_logits(X, Wg):
    """l = X Wg^T, [T, d] x [E, d] -> [T, E]."""
    return X @ Wg.T


def scores(l, score):
    """Per-token expert scores: row softmax, or elementwise sigmoid."""
    if score == "softmax":
        return softmax_rows(l)
    if score == "sigmoid":
        return sigmoid(l)
    raise ValueError(score)


def aux_probs(l, score):
    """q, the router probabilities the aux loss averages (R4)."""
    s = scores(l, score)
    if score == "sigmoid":
        s = s / s.sum(axis=1, keepdims=True)
    return s


def selection_values(l, score, e_bias=None, group_score="max"):
    """What selection ranks: the logits (R2), or fp32 scores plus the bias (R17, R18).

    With no bias and the max group score the logits are ranked exactly.
    Otherwise every score is rounded once to fp32 and the fp32 bias is added
    with one fp32 addition.
    """
    if e_bias is None and group_score == "max":
        return l
    v = scores(l, score).astype(np.float32)
    if e_bias is not None:
        v = (v + np.asarray(e_bias, dtype=np.float32)[None, :]).astype(np.float32)
    return v


def select_topk(l, k, n_groups=1, topk_groups=1, group_score="max"):
    """Group-limited top-k on the values l (logits, or selection_values) (R1, R2, R18).

    Groups are consecutive blocks of E / n_groups experts.  A group's score is
    its largest member value (R1), or the sum of its two largest (R18); the
    topk_groups groups first in the order (-score, group id) stay eligible.
    Eligible experts are ordered by (-value, expert id) and the first k are
    returned in that order.
    """
    T, E = l.shape
    gsize = E // n_groups
    eligible = np.ones((T, E), dtype=bool)
    if n_groups > 1:
        blocks = l.reshape(T, n_groups, gsize)
        if group_score == "max":
            gscore = blocks.max(axis=2)
        elif group_score == "top2":
            top2 = np.sort(blocks, axis=2)[:, :, -2:]
            gscore = top2[:, :, 1] + top2[:, :, 0]
        else:
            raise ValueError(group_score)
        gid = np.broadcast_to(np.arange(n_groups), (T, n_groups))
        kept = np.zeros((T, n_groups), dtype=bool)
        for t in range(T):
            order = np.lexsort((gid[t], -gscore[t]))
            kept[t, order[:topk_groups]] = True
        eligible = np.repeat(kept, gsize, axis=1)
    eid = np.arange(E)
    idx = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        order = np.lexsort((eid, -l[t], ~eligible[t]))
        idx[t] = order[:k]
    return idx


def gate_weights(l, topk_idx, score, route_scale=1.0):
    """g_ti = c * w_ti / sum_j w_tj, w the selected experts' unbiased scores (R3, R17, R19)."""
    w = np.take_along_axis(scores(l, score), topk_idx, axis=1)
    return route_scale * w / w.sum(axis=1, keepdims=True), w


# ----------------------------------------------------------------------------
# Part 4 dispatch and combine
# [Outline] Part 4 "Token Dispatch and Combine": count tokens per expert,
#           slot offsets, gather into per-expert buffers, scatter gradients
#           back, gate-weighted combine with backward.
# [InfraLab] "Project status": expert-major rows with an offsets vector, no
#           capacity padding, empty experts handled.
# ----------------------------------------------------------------------------


@dataclass
class Routing:
    topk_idx: np.ndarray   # [T, k] int64
    counts: np.ndarray     # [E]
    offsets: np.ndarray    # [E + 1], exclusive scan of counts
    slot_of: np.ndarray    # [T, k]   row of (t, i) in the expert-major buffer
    token_of: np.ndarray   # [T * k]  token of each expert-major row
    src_k: np.ndarray = None  # [T * k]  pick index i of each expert-major row


def routing_tables(topk_idx, E):
    """Histogram, exclusive scan and the stable slot map (R7).

    slot_of[t, i] = offsets[e] + #{t' < t : e in topk_idx[t']} for
    e = topk_idx[t, i]: a stable counting sort of the row-major (t, i) list by
    expert.  token_of and src_k invert it: row p holds pick src_k[p] of token
    token_of[p].
    """
    T, k = topk_idx.shape
    flat = topk_idx.reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")          # (t, i) positions by expert
    slot_flat = np.empty(T * k, dtype=np.int64)
    slot_flat[order] = np.arange(T * k)
    token_of = order // k
    src_k = order % k                               # (t, i) = divmod of the row-major position
    return Routing(topk_idx, counts, offsets, slot_flat.reshape(T, k), token_of, src_k)


def gather_rows(X, token_of):
    """Expert-major rows: Xp[p] = X[token_of[p]]."""
    return X[token_of]


def combine(EO, slot_of, gates):
    """Y_t = sum_i g_ti * EO[slot_of[t, i]]."""
    return np.einsum("tk,tkd->td", gates, EO[slot_of])


def combine_backward(dY, EO, slot_of, gates):
    """dg_ti = <dY_t, EO[slot_of[t,i]]>;  dEO[slot_of[t,i]] = g_ti dY_t."""
    dgate = np.einsum("td,tkd->tk", dY, EO[slot_of])
    dEO = np.zeros_like(EO)
    T, k = slot_of.shape
    for i in range(k):
        dEO[slot_of[:, i]] = gates[:, i:i + 1] * dY
    return dgate, dEO


def scatter_rows(dXp, slot_of):
    """dX_t = sum_i dXp[slot_of[t, i]]."""
    return dXp[slot_of].sum(axis=1)


# ----------------------------------------------------------------------------
# Part 5 expert MLP forward and backward
# [Outline] Part 5 "Expert MLP Forward and Backward": up/down projections,
#           biases, activation, backward for inputs, weights and biases.
# [Lesson29] the expert MLP on each expert's slice of tokens.
# [InfraLab] "Numerical contracts": experts in the SwiGLU form
#           W2(SiLU(W1 x) * W3 x).
# ----------------------------------------------------------------------------


def expert_forward(kind, Xp, W1, b1, W2, b2, W3):
    """One expert on its rows.  Returns a dict of the saved intermediates.

    MLP:    H = Xp W1^T + b1, A = act(H), EO = A W2^T + b2.
    SwiGLU: H1 = Xp W1^T, H3 = Xp W3^T, A = silu(H1) * H3, EO = A W2^T.
    """
    if kind == "swiglu":
        H1 = Xp @ W1.T
        H3 = Xp @ W3.T
        A = silu(H1) * H3
        return {"H1": H1, "H3": H3, "A": A, "EO": A @ W2.T}
    act, _ = ACT[kind]
    H = Xp @ W1.T + b1
    A = act(H)
    return {"H": H, "A": A, "EO": A @ W2.T + b2}


def expert_backward(kind, Xp, W1, W2, W3, saved, dEO):
    """Gradients of one expert from dEO on its rows.

    MLP:    db2 = sum dEO, dW2 = dEO^T A, dA = dEO W2, dH = dA * act'(H),
            db1 = sum dH, dW1 = dH^T Xp, dXp = dH W1.
    SwiGLU: dW2 = dEO^T A, dA = dEO W2, dH1 = dA * H3 * silu'(H1),
            dH3 = dA * silu(H1), dW1 = dH1^T Xp, dW3 = dH3^T Xp,
            dXp = dH1 W1 + dH3 W3.
    With no rows every sum is empty, so every gradient is exactly zero (R9).
    """
    A = saved["A"]
    g = {"dW2": dEO.T @ A}
    dA = dEO @ W2
    if kind == "swiglu":
        H1, H3 = saved["H1"], saved["H3"]
        dH1 = dA * H3 * silu_grad(H1)
        dH3 = dA * silu(H1)
        g["dW1"] = dH1.T @ Xp
        g["dW3"] = dH3.T @ Xp
        g["dXp"] = dH1 @ W1 + dH3 @ W3
        g["dH1"], g["dH3"] = dH1, dH3
    else:
        _, act_grad = ACT[kind]
        dH = dA * act_grad(saved["H"])
        g["db2"] = dEO.sum(axis=0)
        g["db1"] = dH.sum(axis=0)
        g["dW1"] = dH.T @ Xp
        g["dXp"] = dH @ W1
        g["dH"] = dH
    g["dA"] = dA
    return g


# ----------------------------------------------------------------------------
# Part 6 load-balancing aux loss, Part 7 loss and optimiser
# [Outline] Part 6 "Load Balancing Auxiliary Loss": dispatch fractions, mean
#           router probabilities, the aux loss, gradient to the probabilities.
# [Outline] Part 7 "Loss, Optimizer, and Training Loop": MSE, gradient
#           zeroing, SGD.
# ----------------------------------------------------------------------------


def aux_loss(counts, q, k):
    """aux = E * sum_e f_e P_e (R4).  Returns (aux, f, P)."""
    T, E = q.shape
    f = counts / float(T * k)
    P = q.mean(axis=0)
    return E * float(np.dot(f, P)), f, P


def aux_grad_q(counts, T, k, E, aux_coef):
    """d(aux_coef * aux)/dq_te = aux_coef * E * f_e / T, the same for all t."""
    f = counts / float(T * k)
    return np.broadcast_to(aux_coef * E * f / T, (T, E))


def mse(Y, Yt):
    """Mean of (Y - Yt)^2 over all elements (R5), and its gradient."""
    n = Y.size
    r = Y - Yt
    return float((r * r).sum() / n), 2.0 * r / n


def renorm_backward(dgate, gates, w, route_scale=1.0):
    """dw_i = (c dg_i - sum_j g_j dg_j) / S with S = sum_j w_j and g = c w / S (R19)."""
    S = w.sum(axis=1, keepdims=True)
    return (route_scale * dgate - (gates * dgate).sum(axis=1, keepdims=True)) / S


def router_backward(l, topk_idx, dw, dq, score):
    """dl from the selected-score gradient dw [T,k] and the aux gradient dq [T,E].

    softmax: dp = dq + scatter(dw); dl = p * (dp - <dp, p>).
    sigmoid: ds = scatter(dw) + (dq - <dq, q>) / Z, Z = sum_e s_e;
             dl = ds * s * (1 - s).
    """
    T, E = l.shape
    sel = np.zeros((T, E))
    np.put_along_axis(sel, topk_idx, dw, axis=1)
    if score == "softmax":
        p = softmax_rows(l)
        dp = dq + sel
        return p * (dp - (dp * p).sum(axis=1, keepdims=True))
    s = sigmoid(l)
    Z = s.sum(axis=1, keepdims=True)
    q = s / Z
    ds = sel + (dq - (dq * q).sum(axis=1, keepdims=True)) / Z
    return ds * s * (1.0 - s)


def sgd(theta, grad, lr):
    """theta - lr * grad (R10)."""
    return theta - lr * grad


# ----------------------------------------------------------------------------
# The whole layer
# ----------------------------------------------------------------------------


@dataclass
class Shape:
    E: int
    k: int
    n_groups: int = 1
    topk_groups: int = 1
    score: str = "softmax"
    expert: str = "relu"
    group_score: str = "max"      # R1 or R18
    route_scale: float = 1.0      # R19


def route(X, Wg, shp: Shape, topk_idx=None, e_bias=None):
    """Router + selection + gates + routing tables.

    topk_idx may be supplied by the caller (a resolved routing, see the
    parity tests); it must be a valid top-k of these logits up to the logit
    error of the device arithmetic.  e_bias is the optional correction bias
    (R17).
    """
    l = router_logits(X, Wg)
    if topk_idx is None:
        v = selection_values(l, shp.score, e_bias, shp.group_score)
        topk_idx = select_topk(v, shp.k, shp.n_groups, shp.topk_groups, group_score=shp.group_score)
    g, w = gate_weights(l, topk_idx, shp.score, shp.route_scale)
    r = routing_tables(topk_idx, shp.E)
    return {"logits": l, "topk_idx": topk_idx, "gates": g, "w": w, "routing": r,
            "q": aux_probs(l, shp.score)}


def shared_forward(X, P):
    """Shared branch (R20): one SwiGLU with weights Ws1, Ws3, Ws2 over every token."""
    return expert_forward("swiglu", X, P["Ws1"], None, P["Ws2"], None, P["Ws3"])


def shared_backward(X, P, saved, dY):
    """Gradients of the shared branch: its output enters Y with no gate, so the
    upstream gradient is dY itself (R20)."""
    g = expert_backward("swiglu", X, P["Ws1"], P["Ws2"], P["Ws3"], saved, dY)
    return {"dWs1": g["dW1"], "dWs2": g["dW2"], "dWs3": g["dW3"], "dX": g["dXp"]}


# trained parameters: router, routed experts, shared branch (R20)
PARAM_NAMES = ("Wg", "W1", "b1", "W2", "b2", "W3", "Ws1", "Ws2", "Ws3")


def layer_forward(X, P: Dict[str, Optional[np.ndarray]], shp: Shape, topk_idx=None):
    """Forward of the whole layer.  P holds Wg, W1, b1, W2, b2, W3 (float64),
    optionally the shared branch Ws1, Ws2, Ws3 (R20), and optionally e_bias, the
    correction bias (R17), which no gradient reaches."""
    fw = route(X, P["Wg"], shp, topk_idx, P.get("e_bias"))
    r = fw["routing"]
    T, d = X.shape
    EO = np.zeros((T * shp.k, d))
    saved = []
    for e in range(shp.E):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        Xp = gather_rows(X, r.token_of[lo:hi])
        s = expert_forward(shp.expert, Xp, P["W1"][e], None if P.get("b1") is None else P["b1"][e],
                           P["W2"][e], None if P.get("b2") is None else P["b2"][e],
                           None if P.get("W3") is None else P["W3"][e])
        EO[lo:hi] = s["EO"]
        saved.append(s)
    fw["EO"] = EO
    fw["saved"] = saved
    fw["Y"] = combine(EO, r.slot_of, fw["gates"])
    if P.get("Ws1") is not None:                # shared branch over every token (R20)
        fw["shared"] = shared_forward(X, P)
        fw["Y"] = fw["Y"] + fw["shared"]["EO"]
    aux, f, Pm = aux_loss(r.counts, fw["q"], shp.k)
    fw["aux"], fw["f"], fw["P"] = aux, f, Pm
    return fw


def layer_backward(X, P, shp: Shape, fw, dY, aux_coef):
    """Full backward from dY (and aux_coef * aux).  Returns every gradient."""
    r = fw["routing"]
    T, d = X.shape
    E = shp.E
    dgate, dEO = combine_backward(dY, fw["EO"], r.slot_of, fw["gates"])
    grads = {"dW1": np.zeros_like(P["W1"]), "dW2": np.zeros_like(P["W2"])}
    if P.get("W3") is not None:
        grads["dW3"] = np.zeros_like(P["W3"])
    if P.get("b1") is not None:
        grads["db1"] = np.zeros_like(P["b1"])
        grads["db2"] = np.zeros_like(P["b2"])
    dXp = np.zeros((T * shp.k, d))
    for e in range(E):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        Xp = gather_rows(X, r.token_of[lo:hi])
        g = expert_backward(shp.expert, Xp, P["W1"][e], P["W2"][e],
                            None if P.get("W3") is None else P["W3"][e],
                            fw["saved"][e], dEO[lo:hi])
        for n in ("dW1", "dW2", "dW3", "db1", "db2"):
            if n in g:
                grads[n][e] = g[n]
        dXp[lo:hi] = g["dXp"]
    dX = scatter_rows(dXp, r.slot_of)
    if P.get("Ws1") is not None:                # shared branch: upstream gradient dY (R20)
        gs = shared_backward(X, P, fw["shared"], dY)
        grads["dWs1"], grads["dWs2"], grads["dWs3"] = gs["dWs1"], gs["dWs2"], gs["dWs3"]
        dX = dX + gs["dX"]
    dw = renorm_backward(dgate, fw["gates"], fw["w"], shp.route_scale)
    dq = aux_grad_q(r.counts, T, shp.k, E, aux_coef)
    dl = router_backward(fw["logits"], r.topk_idx, dw, dq, shp.score)
    grads["dWg"] = dl.T @ X
    grads["dX"] = dX + dl @ P["Wg"]
    grads["dlogits"] = dl
    grads["dgate"] = dgate
    return grads


def train_step(X, Yt, P, shp: Shape, lr, aux_coef, topk_idx=None):
    """Forward, MSE + aux_coef * aux (R11), backward, SGD on every parameter."""
    fw = layer_forward(X, P, shp, topk_idx)
    m, dY = mse(fw["Y"], Yt)
    loss = m + aux_coef * fw["aux"]
    grads = layer_backward(X, P, shp, fw, dY, aux_coef)
    newP = {"e_bias": P.get("e_bias")}          # the correction bias is not trained (R17)
    for n in PARAM_NAMES:
        newP[n] = None if P.get(n) is None else sgd(P[n], grads["d" + n], lr)
    return {"fw": fw, "grads": grads, "mse": m, "loss": loss, "params": newP, "dY": dY}


def train_step_streamed(X, Yt, Wg, get_expert, shp: Shape, lr, aux_coef, topk_idx=None,
                        e_bias=None, keep=(), dY=None, progress=None):
    """train_step for a layer whose expert weights do not fit in memory at once.

    The steps and their order are those of train_step (route, experts, combine,
    MSE + aux_coef * aux, backward, SGD), with two differences of bookkeeping
    only: the expert weights are fetched one expert at a time, by
    get_expert(e) -> {"W1", "W2", "W3" (SwiGLU), "b1", "b2" (MLP)} in float64,
    once for the forward and once for the backward; and the combine backward
    is taken per expert segment (dg_ti = <dY_t, EO[slot]> and
    dEO[slot] = g_ti dY_t for the rows of that segment), so that dEO never
    exists as a whole.  dX is summed in pick order as in scatter_rows.
    With dY given, the backward starts from it instead of the MSE gradient
    (the loss is still reported).  Returns the loss parts, Y, dY, dX, dWg, the
    routing, and for each expert in `keep` its gradients and updated weights;
    the router weight's update is Wg - lr * dWg.  progress, if given, is called
    with a short text after every 32 experts of each pass.
    """
    fw = route(X, Wg, shp, topk_idx, e_bias)
    r = fw["routing"]
    T, d = X.shape
    k, E = shp.k, shp.E
    gates = fw["gates"]
    gate_row = gates.reshape(-1)[r.token_of * k + r.src_k]      # g of each expert-major row
    EO = np.zeros((T * k, d))
    saved = {}
    for e in range(E):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        if hi == lo:
            continue
        p = get_expert(e)
        s = expert_forward(shp.expert, gather_rows(X, r.token_of[lo:hi]), p["W1"], p.get("b1"),
                           p["W2"], p.get("b2"), p.get("W3"))
        EO[lo:hi] = s.pop("EO")
        saved[e] = s
        if progress and (e + 1) % 32 == 0:
            progress(f"oracle forward: {e + 1} of {E} experts")
    Y = combine(EO, r.slot_of, gates)
    aux, f, Pm = aux_loss(r.counts, fw["q"], k)
    m, dY_mse = mse(Y, Yt)
    if dY is None:
        dY = dY_mse
    dgate = np.zeros((T, k))
    dXp = np.zeros((T * k, d))
    out = {"experts": {}}
    for e in range(E):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        if hi == lo and e not in keep:
            continue
        p = get_expert(e)
        tok = r.token_of[lo:hi]
        EOe = EO[lo:hi]
        dgate[tok, r.src_k[lo:hi]] = (dY[tok] * EOe).sum(axis=1)
        dEO = gate_row[lo:hi, None] * dY[tok]
        if hi == lo:
            s = {"A": np.zeros((0, p["W2"].shape[1])), "H": np.zeros((0, p["W1"].shape[0])),
                 "H1": np.zeros((0, p["W1"].shape[0])), "H3": np.zeros((0, p["W1"].shape[0]))}
        else:
            s = saved.pop(e)
        g = expert_backward(shp.expert, gather_rows(X, tok), p["W1"], p["W2"], p.get("W3"), s, dEO)
        dXp[lo:hi] = g["dXp"]
        if e in keep:
            ge = {n: g[n] for n in ("dW1", "dW2", "dW3", "db1", "db2") if n in g}
            new = {n[1:]: sgd(p[n[1:]], ge[n], lr) for n in ge}
            out["experts"][e] = {"grads": ge, "params": new}
        if progress and (e + 1) % 32 == 0:
            progress(f"oracle backward: {e + 1} of {E} experts")
    del EO, saved
    dX = scatter_rows(dXp, r.slot_of)
    del dXp
    dw = renorm_backward(dgate, gates, fw["w"], shp.route_scale)
    dq = aux_grad_q(r.counts, T, k, E, aux_coef)
    dl = router_backward(fw["logits"], r.topk_idx, dw, dq, shp.score)
    out.update({"mse": m, "aux": aux, "loss": m + aux_coef * aux, "Y": Y, "dY": dY,
                "dX": dX + dl @ Wg, "dWg": dl.T @ X, "dgate": dgate, "dlogits": dl,
                "logits": fw["logits"], "gates": gates, "routing": r})
    return out
