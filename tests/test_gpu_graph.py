"""The library's launches can be captured into a HIP graph and replayed.

Every entry point only launches kernels on the caller's stream (no allocation,
copy, memset or synchronisation), so a whole forward + backward, or a whole
training step, is captured as it is.  Each replay is checked bit for bit
against the eager result, with eager work (the outputs overwritten) between
the replays.
"""
import pytest
import torch

from sparse_mixture_experts_gate_amd import _lib as L
from sparse_mixture_experts_gate_amd import workloads as W
from tests.gpu_harness import LayerRun, say
from tests.test_gpu_layer import BF16_CASES, F32_CASES, PARAM_NAMES, SHARED_CASES

pytestmark = pytest.mark.gpu

CASES = [F32_CASES[2], BF16_CASES[0], SHARED_CASES[2]]


def _outputs(run):
    return {"Y": run.Y.clone(), **{"r_" + n: v.clone() for n, v in run.routing.items()},
            **{"g_" + n: v.clone() for n, v in run.grads.items()}}


def _clobber(run):
    run.Y.fill_(float("nan"))
    for v in run.routing.values():
        v.fill_(-7)
    for v in run.grads.values():
        v.fill_(float("nan"))


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_forward_backward_graph_replays_match_eager(w):
    inp = W.make_inputs(w, masters=True)
    dY = W.make_upstream_grad(w).cuda()
    run = LayerRun(w, inp)
    run.forward()
    run.backward(dY, 0.2)
    torch.cuda.synchronize()
    ref = _outputs(run)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        L.moe_forward(run.cfg, run.X, run.weights, run.Y, run.routing, run.ws, stream=s)
        L.moe_backward(run.cfg, run.X, run.weights, run.routing, dY, 0.2, run.grads, run.ws, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        _clobber(run)                      # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(run)
        for n in ref:
            assert torch.equal(got[n], ref[n]), (rep, n)
    say(f"[{w.name}] 3 graph replays equal the eager forward + backward")


@pytest.mark.parametrize("w", [BF16_CASES[0], SHARED_CASES[3]], ids=lambda w: w.name)
@pytest.mark.parametrize("fused", [False, True], ids=["stored", "fused"])
def test_train_step_graph_matches_eager_steps(w, fused):
    """Three replays of a captured training step move the parameters exactly as
    three eager steps do."""
    inp = W.make_inputs(w, masters=True)
    dev = "cuda"

    def setup():
        cfg = L.config(w)
        st = {"cfg": cfg, "ws": L.alloc_workspace(cfg, dev), "r": L.alloc_routing(w, dev),
              "g": L.alloc_grads(w, dev), "Y": torch.empty(w.T, w.d, dtype=w.torch_dtype, device=dev),
              "loss": torch.empty(3, dtype=torch.float32, device=dev),
              "X": inp["X"].to(dev), "Yt": inp["Yt"].to(dev), "p": {}}
        if fused:
            for n in ("dW1", "dW2", "dW3", "dWs1", "dWs2", "dWs3"):
                st["g"].pop(n, None)
        for n in PARAM_NAMES:
            if inp.get(n) is not None:
                st["p"][n] = inp[n].clone().to(dev)
                st["p"][n + "_w"] = inp[n + "_w"].clone().to(dev)
        return st

    def step(st, stream=None):
        L.moe_train_step(st["cfg"], st["X"], st["Yt"], st["p"], w.lr, w.aux_coef, st["Y"], st["r"],
                         st["g"], st["loss"], st["ws"], stream=stream)

    eager, graphed = setup(), setup()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    snapshot = {n: v.clone() for n, v in graphed["p"].items()}
    with torch.cuda.graph(g, stream=s):
        step(graphed, stream=s)
    torch.cuda.synchronize()
    # capture does not execute: the parameters are untouched until the first replay
    for n, v in snapshot.items():
        assert torch.equal(graphed["p"][n], v), n
    for rep in range(3):
        step(eager)
        graphed["Y"].fill_(float("nan"))           # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(graphed["loss"], eager["loss"]), rep
        assert torch.equal(graphed["Y"], eager["Y"]), rep
        for n in eager["p"]:
            assert torch.equal(graphed["p"][n], eager["p"][n]), (rep, n)
