"""Workload shapes and seeded synthetic inputs for the sparse MoE layer.

This module holds no arithmetic of the method: it only names the five layer
shapes and draws their inputs.  Both the HIP path and the float64 oracle take
their inputs from here, so the two sides always see the same values.

Recipe (every tensor has its own seed, derived from one base seed):
  * X, Y_target ~ N(0, 1), drawn in float32.
  * Router weight Wg [E, d] ~ N(0, variance 1/d).  The skewed workload scales
    row e by (e+1)^-1.2 (a Zipf(1.2) profile of logit spread) and makes rows
    25..31 exact copies of row 25, so that ties on the smaller expert id leave
    experts 29, 30 and 31 with no rows at all.
  * Expert weights ~ N(0, variance 1/fan_in) (W1, W3: fan_in = d; W2: fan_in =
    ffn), except the largest workload, whose expert weights have standard
    deviation 0.02.  Biases start at zero.
  * float32 draws are the master copies; bfloat16 working copies are their
    round-to-nearest-even conversion (torch's ``.to(torch.bfloat16)``).

Inputs are drawn with torch's generator on the device asked for.  CPU and GPU
generators give different streams, so a test that needs host copies of
GPU-drawn inputs copies them back; it never redraws them.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    ffn: int
    k: int
    n_groups: int
    topk_groups: int
    score: str        # "softmax" | "sigmoid"
    expert: str       # "relu" | "gelu" | "swiglu"
    dtype: str        # "f32" | "bf16"
    lr: float
    aux_coef: float
    steps: int
    init: str         # "fan_in" | "std0.02"
    gate: str         # "normal" | "zipf_tie"
    # router variants (defaults: the plain gate)
    group_score: str = "max"      # "max" | "top2"
    route_scale: float = 1.0
    e_bias: float = 0.0           # std of the seeded correction bias; 0 = no bias
    n_shared: int = 0             # shared experts: one SwiGLU of hidden n_shared * ffn; 0 = none
    fused_dispatch: int = 0       # 1: expert contractions read X / dY through token_of (SwiGLU bf16)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def has_bias(self) -> bool:
        return self.expert in ("relu", "gelu")

    @property
    def rows(self) -> int:
        return self.T * self.k

    def expert_gemm_flops(self) -> float:
        """Ideal active-row flops of the expert contractions, forward only."""
        m = 3 if self.expert == "swiglu" else 2
        return 2.0 * self.T * self.k * self.d * self.ffn * m

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = [
    Workload("tiny_f32_relu_t64", T=64, d=32, E=4, ffn=64, k=2, n_groups=1, topk_groups=1,
             score="softmax", expert="relu", dtype="f32", lr=1e-2, aux_coef=0.01, steps=1,
             init="fan_in", gate="normal"),
    Workload("gelu_mlp_t4096_d1024_e8", T=4096, d=1024, E=8, ffn=4096, k=2, n_groups=1,
             topk_groups=1, score="softmax", expert="gelu", dtype="bf16", lr=1e-3,
             aux_coef=0.01, steps=20, init="fan_in", gate="normal"),
    Workload("skewed_swiglu_t8192_e32", T=8192, d=1024, E=32, ffn=2816, k=4, n_groups=1,
             topk_groups=1, score="softmax", expert="swiglu", dtype="bf16", lr=1e-3,
             aux_coef=0.01, steps=1, init="fan_in", gate="zipf_tie"),
    Workload("grouped_sigmoid_t16384_e64", T=16384, d=2048, E=64, ffn=1408, k=6, n_groups=8,
             topk_groups=4, score="sigmoid", expert="swiglu", dtype="bf16", lr=1e-3,
             aux_coef=0.01, steps=1, init="fan_in", gate="normal"),
    Workload("grouped_sigmoid_t32768_d7168_e256", T=32768, d=7168, E=256, ffn=2048, k=8,
             n_groups=8, topk_groups=4, score="sigmoid", expert="swiglu", dtype="bf16",
             lr=1e-3, aux_coef=0.01, steps=1, init="std0.02", gate="normal"),
]

BY_NAME = {w.name: w for w in WORKLOADS}

_TENSOR_ID = {"X": 1, "Yt": 2, "Wg": 3, "W1": 4, "W2": 5, "W3": 6, "dY": 7, "logits": 8, "e_bias": 9,
              "Ws1": 10, "Ws2": 11, "Ws3": 12}


def tensor_seed(base: int, tensor: str, expert: int = 0) -> int:
    return (int(base) << 32) + (_TENSOR_ID[tensor] << 20) + int(expert)


def _normal(shape, std: float, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        out.mul_(std)
    return out


def expert_std(w: Workload, which: str) -> float:
    if w.init == "std0.02":
        return 0.02
    fan_in = w.ffn if which == "W2" else w.d
    return fan_in ** -0.5


def make_gate(w: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    """Router weight master copy, float32 [E, d]."""
    if w.gate == "normal":
        return _normal((w.E, w.d), w.d ** -0.5, tensor_seed(seed, "Wg"), device)
    if w.gate == "zipf_tie":
        u = _normal((w.E, w.d), w.d ** -0.5, tensor_seed(seed, "Wg"), device)
        scale = torch.tensor([(e + 1) ** -1.2 for e in range(w.E)], dtype=torch.float32,
                             device=device)
        g = u * scale[:, None]
        tie_from = 25
        g[tie_from + 1:] = g[tie_from]
        return g
    raise ValueError(w.gate)


def make_shared(w: Workload, which: str, seed: int = 0, device="cpu") -> torch.Tensor:
    """A shared-branch master weight, float32: Ws1/Ws3 [Hs, d], Ws2 [d, Hs], Hs = n_shared * ffn;
    initialised like the routed experts (fan-in of the shared hidden width for Ws2)."""
    hs = w.n_shared * w.ffn
    shape = (w.d, hs) if which == "Ws2" else (hs, w.d)
    std = 0.02 if w.init == "std0.02" else (hs if which == "Ws2" else w.d) ** -0.5
    return _normal(shape, std, tensor_seed(seed, which), device)


def make_expert(w: Workload, which: str, e: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """One expert's master weight, float32: W1/W3 [ffn, d], W2 [d, ffn]."""
    shape = (w.d, w.ffn) if which == "W2" else (w.ffn, w.d)
    return _normal(shape, expert_std(w, which), tensor_seed(seed, which, e), device)


def make_inputs(w: Workload, seed: int = 0, device="cpu",
                masters: bool = True) -> Dict[str, Optional[torch.Tensor]]:
    """All inputs of one layer step: activations, targets, master and working weights.

    Returned keys: X, Yt (working dtype); Wg, W1, b1, W2, b2, W3, Ws1, Ws3, Ws2
    (float32 masters; the Ws* are the shared branch, None when w.n_shared == 0);
    the same names with a ``_w`` suffix for the working copies; e_bias, the
    float32 correction bias [E] ~ N(0, w.e_bias^2) (None when w.e_bias == 0).
    Tensors that the expert kind does not use are None.  With masters=False
    the float32 masters are not kept (their keys hold None) and only the
    working copies are built, one expert at a time.
    """
    wd = w.torch_dtype
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["X"] = _normal((w.T, w.d), 1.0, tensor_seed(seed, "X"), device).to(wd)
    out["Yt"] = _normal((w.T, w.d), 1.0, tensor_seed(seed, "Yt"), device).to(wd)
    gate = make_gate(w, seed, device)
    out["Wg"], out["Wg_w"] = (gate if masters else None), gate.to(wd)
    for n in ("W1", "W2", "W3"):
        if n == "W3" and w.expert != "swiglu":
            out[n] = out[n + "_w"] = None
            continue
        shape = (w.E, w.d, w.ffn) if n == "W2" else (w.E, w.ffn, w.d)
        master = torch.empty(shape, dtype=torch.float32, device=device) if masters else None
        work = torch.empty(shape, dtype=wd, device=device)
        for e in range(w.E):
            t = make_expert(w, n, e, seed, device)
            if masters:
                master[e] = t
            work[e] = t.to(wd)
        out[n], out[n + "_w"] = master, work
    if w.has_bias:
        for n, shape in (("b1", (w.E, w.ffn)), ("b2", (w.E, w.d))):
            z = torch.zeros(shape, dtype=torch.float32, device=device)
            out[n], out[n + "_w"] = (z if masters else None), z.to(wd)
    else:
        out["b1"] = out["b2"] = out["b1_w"] = out["b2_w"] = None
    out["e_bias"] = (_normal((w.E,), w.e_bias, tensor_seed(seed, "e_bias"), device)
                     if w.e_bias > 0 else None)
    for n in ("Ws1", "Ws3", "Ws2"):
        if w.n_shared > 0:
            t = make_shared(w, n, seed, device)
            out[n], out[n + "_w"] = (t if masters else None), t.to(wd)
        else:
            out[n] = out[n + "_w"] = None
    return out


def make_upstream_grad(w: Workload, seed: int = 0, device="cpu", scale: float = 1.0,
                       token_mask: Optional[torch.Tensor] = None) -> torch.Tensor:
    """A caller-supplied dY [T, d] ~ N(0, scale^2), optionally zero outside token_mask."""
    g = _normal((w.T, w.d), scale, tensor_seed(seed, "dY"), device)
    if token_mask is not None:
        g = g * token_mask.to(device=device, dtype=torch.float32)[:, None]
    return g.to(w.torch_dtype)


def make_router_logits(T: int, E: int, kind: str, seed: int = 0) -> torch.Tensor:
    """float32 [T, E] logits for routing-only tests (CPU).

    kind: "normal" ~ N(0,1); "ties" small integers in [-3, 3] with about a
    quarter of the zeros negative (so +0.0 and -0.0 meet); "uniform" cyclic
    shifts of 0..E-1 (every expert equally loaded when E divides T).
    """
    g = torch.Generator().manual_seed(tensor_seed(seed, "logits"))
    if kind == "normal":
        return torch.randn(T, E, generator=g)
    if kind == "ties":
        v = torch.randint(-3, 4, (T, E), generator=g).to(torch.float32)
        neg = torch.rand(T, E, generator=g) < 0.25
        v = torch.where((v == 0) & neg, torch.tensor(-0.0), v)
        return v
    if kind == "uniform":
        t = torch.arange(T)[:, None]
        e = torch.arange(E)[None, :]
        return ((e - t) % E).to(torch.float32)
    raise ValueError(kind)
