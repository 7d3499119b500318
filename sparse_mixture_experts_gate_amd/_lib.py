"""ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
torch supplies device memory and the stream.  If the library is missing the
first call raises; nothing falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

SCORE = {"softmax": 0, "sigmoid": 1}
EXPERT = {"relu": 0, "gelu": 1, "swiglu": 2}
DTYPE = {"f32": 0, "bf16": 1}
GROUP = {"max": 0, "top2": 1}
WS = {"XP": 0, "H": 1, "A": 2, "EO": 3}

STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_NULL_PTR", -3: "MOE_ERR_MISALIGNED",
          -4: "MOE_ERR_WORKSPACE", -5: "MOE_ERR_UNSUPPORTED", -6: "MOE_ERR_HIP", -7: "MOE_ERR_SCRATCH"}

EXPORTS = ["moe_workspace_bytes", "moe_workspace_offset", "moe_route", "moe_route_noalloc", "moe_forward",
           "moe_backward", "moe_train_step", "moe_train_step_profiled", "moe_status_string",
           "moe_abi_version"]

STAGES = ["router_logits", "route", "gather", "up_fwd", "down_fwd", "shared_fwd", "combine_loss",
          "combine_bwd", "down_dgrad", "down_wgrad", "up_dgrad", "up_wgrad", "shared_bwd", "bias_grads",
          "router_bwd", "router_dwg", "router_dx", "scatter", "sgd"]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")


class moe_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "d", "E", "ffn", "k", "n_groups", "topk_groups", "score", "expert", "dtype",
                 "group_score")] + [("route_scale", ctypes.c_float), ("n_shared", ctypes.c_int32),
                                    ("fused_dispatch", ctypes.c_int32)]


WEIGHTS = ("Wg", "W1", "b1", "W2", "b2", "W3", "e_bias", "Ws1", "Ws3", "Ws2")
PARAMS = ("Wg", "W1", "b1", "W2", "b2", "W3", "Wg_w", "W1_w", "b1_w", "W2_w", "b2_w", "W3_w", "e_bias",
          "Ws1", "Ws3", "Ws2", "Ws1_w", "Ws3_w", "Ws2_w")
GRADS = ("dX", "dWg", "dW1", "db1", "dW2", "db2", "dW3", "dWs1", "dWs3", "dWs2")


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHTS]


ROUTING = ("logits", "topk_idx", "gates", "counts", "offsets", "slot_of", "token_of", "aux", "src_k")


class moe_routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ROUTING]


class moe_grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRADS]


class moe_params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in PARAMS]


_lib = None
ABI_VERSION = 5                 # the structs above, as include/moe.h declares them


def load() -> ctypes.CDLL:
    """Load libmoe.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_mixture_experts_gate_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        lib.moe_workspace_bytes.argtypes = [P(moe_config)]
        lib.moe_workspace_bytes.restype = ctypes.c_size_t
        lib.moe_workspace_offset.argtypes = [P(moe_config), ctypes.c_int32]
        lib.moe_workspace_offset.restype = ctypes.c_int64
        lib.moe_route.argtypes = [P(moe_config), ctypes.c_void_p, ctypes.c_void_p, P(moe_routing),
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.moe_route_noalloc.argtypes = [P(moe_config), ctypes.c_void_p, ctypes.c_void_p, P(moe_routing),
                                          ctypes.c_void_p]
        lib.moe_forward.argtypes = [P(moe_config), ctypes.c_void_p, P(moe_weights), ctypes.c_void_p,
                                    P(moe_routing), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.moe_backward.argtypes = [P(moe_config), ctypes.c_void_p, P(moe_weights), P(moe_routing),
                                     ctypes.c_void_p, ctypes.c_float, P(moe_grads), ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]
        lib.moe_train_step.argtypes = [P(moe_config), ctypes.c_void_p, ctypes.c_void_p, P(moe_params),
                                       ctypes.c_float, ctypes.c_float, ctypes.c_void_p, P(moe_routing),
                                       P(moe_grads), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
        lib.moe_train_step_profiled.argtypes = lib.moe_train_step.argtypes + [ctypes.c_void_p]
        for f in ("moe_route", "moe_route_noalloc", "moe_forward", "moe_backward", "moe_train_step",
                  "moe_train_step_profiled"):
            getattr(lib, f).restype = ctypes.c_int
        lib.moe_status_string.argtypes = [ctypes.c_int]
        lib.moe_status_string.restype = ctypes.c_char_p
        lib.moe_abi_version.argtypes = []
        lib.moe_abi_version.restype = ctypes.c_int32
        if lib.moe_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {lib.moe_abi_version()}, this binding "
                               f"expects {ABI_VERSION}: rebuild it")
        _lib = lib
    return _lib


# ---- marshalling helpers ------------------------------------------------------------

def config(w, group_score=None, route_scale=None) -> moe_config:
    """moe_config from a workloads.Workload (or anything with the same fields).

    group_score ("max" / "top2" or the MOE_GROUP_* code) and route_scale default
    to the workload's own fields when it has them, else to the plain gate.
    """
    def code(table, v):
        return table[v] if isinstance(v, str) else int(v)
    gs = group_score if group_score is not None else getattr(w, "group_score", "max")
    rs = route_scale if route_scale is not None else getattr(w, "route_scale", 1.0)
    return moe_config(w.T, w.d, w.E, w.ffn, w.k, w.n_groups, w.topk_groups, code(SCORE, w.score),
                      code(EXPERT, w.expert), code(DTYPE, w.dtype), code(GROUP, gs), float(rs),
                      int(getattr(w, "n_shared", 0)), int(getattr(w, "fused_dispatch", 0)))


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def status_string(status: int) -> str:
    return load().moe_status_string(status).decode()


def _check(status: int, what: str):
    if status != 0:
        raise MoeError(status, what)


def workspace_bytes(cfg: moe_config) -> int:
    return load().moe_workspace_bytes(ctypes.byref(cfg))


def workspace_offset(cfg: moe_config, which: str) -> int:
    return load().moe_workspace_offset(ctypes.byref(cfg), WS[which])


def abi_version() -> int:
    return load().moe_abi_version()


def routing_struct(r: dict) -> moe_routing:
    return moe_routing(*[_p(r.get(n)) for n in ROUTING])


def weights_struct(w: dict) -> moe_weights:
    return moe_weights(*[_p(w.get(n)) for n in WEIGHTS])


def grads_struct(g: dict) -> moe_grads:
    return moe_grads(*[_p(g.get(n)) for n in GRADS])


def params_struct(p: dict) -> moe_params:
    return moe_params(*[_p(p.get(n)) for n in PARAMS])


# ---- entry points, same names as the C ABI -----------------------------------------

def moe_route(cfg: moe_config, logits: torch.Tensor, routing: dict, workspace: torch.Tensor,
              stream=None, e_bias: Optional[torch.Tensor] = None) -> None:
    r = routing_struct(routing)
    _check(load().moe_route(ctypes.byref(cfg), _p(logits), _p(e_bias), ctypes.byref(r), _p(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream)), "moe_route")


def moe_route_noalloc(cfg: moe_config, logits: torch.Tensor, routing: dict, stream=None,
                      e_bias: Optional[torch.Tensor] = None) -> None:
    r = routing_struct(routing)
    _check(load().moe_route_noalloc(ctypes.byref(cfg), _p(logits), _p(e_bias), ctypes.byref(r),
                                    _stream(stream)), "moe_route_noalloc")


def moe_forward(cfg: moe_config, X: torch.Tensor, weights: dict, Y: torch.Tensor, routing: dict,
                workspace: torch.Tensor, stream=None) -> None:
    w = weights_struct(weights)
    r = routing_struct(routing)
    _check(load().moe_forward(ctypes.byref(cfg), _p(X), ctypes.byref(w), _p(Y), ctypes.byref(r),
                              _p(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream)), "moe_forward")


def moe_backward(cfg: moe_config, X: torch.Tensor, weights: dict, routing: dict, dY: torch.Tensor,
                 aux_coef: float, grads: dict, workspace: torch.Tensor, stream=None) -> None:
    w = weights_struct(weights)
    r = routing_struct(routing)
    g = grads_struct(grads)
    _check(load().moe_backward(ctypes.byref(cfg), _p(X), ctypes.byref(w), ctypes.byref(r), _p(dY),
                               ctypes.c_float(aux_coef), ctypes.byref(g), _p(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)),
           "moe_backward")


def moe_train_step(cfg: moe_config, X: torch.Tensor, Y_target: torch.Tensor, params: dict, lr: float,
                   aux_coef: float, Y: torch.Tensor, routing: dict, grads: dict, loss_out: torch.Tensor,
                   workspace: torch.Tensor, stream=None) -> None:
    p = params_struct(params)
    r = routing_struct(routing)
    g = grads_struct(grads)
    _check(load().moe_train_step(ctypes.byref(cfg), _p(X), _p(Y_target), ctypes.byref(p),
                                 ctypes.c_float(lr), ctypes.c_float(aux_coef), _p(Y), ctypes.byref(r),
                                 ctypes.byref(g), _p(loss_out), _p(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "moe_train_step")


class StageEvents:
    """MOE_NUM_STAGES + 1 hipEvents (created through the HIP runtime) for
    moe_train_step_profiled, and the per-stage elapsed times they record."""

    def __init__(self):
        # the SONAME resolves to the HIP runtime already loaded by torch (one runtime per process)
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        n = len(STAGES) + 1
        self.array = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.array[i] = ev
        self.ms = {s: [] for s in STAGES}

    def collect(self):
        """Read the stage times of the last profiled call (its stream must be synchronised)."""
        for i, name in enumerate(STAGES):
            t = ctypes.c_float()
            if self.hip.hipEventElapsedTime(ctypes.byref(t), self.array[i], self.array[i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            self.ms[name].append(t.value)

    def __del__(self):
        try:
            for ev in self.array:
                self.hip.hipEventDestroy(ev)
        except Exception:
            pass


def moe_train_step_profiled(cfg: moe_config, X: torch.Tensor, Y_target: torch.Tensor, params: dict,
                            lr: float, aux_coef: float, Y: torch.Tensor, routing: dict, grads: dict,
                            loss_out: torch.Tensor, workspace: torch.Tensor, events: StageEvents,
                            stream=None) -> None:
    p = params_struct(params)
    r = routing_struct(routing)
    g = grads_struct(grads)
    _check(load().moe_train_step_profiled(
        ctypes.byref(cfg), _p(X), _p(Y_target), ctypes.byref(p), ctypes.c_float(lr),
        ctypes.c_float(aux_coef), _p(Y), ctypes.byref(r), ctypes.byref(g), _p(loss_out),
        _p(workspace), workspace.numel() * workspace.element_size(), _stream(stream),
        ctypes.cast(events.array, ctypes.c_void_p)), "moe_train_step_profiled")


# ---- buffer allocation (torch is the allocator) ----------------------------------------

def alloc_routing(w, device) -> dict:
    T, E, k = w.T, w.E, w.k
    i32, f32 = torch.int32, torch.float32
    return {"logits": torch.empty(T, E, dtype=f32, device=device),
            "topk_idx": torch.empty(T, k, dtype=i32, device=device),
            "gates": torch.empty(T, k, dtype=f32, device=device),
            "counts": torch.empty(E, dtype=i32, device=device),
            "offsets": torch.empty(E + 1, dtype=i32, device=device),
            "slot_of": torch.empty(T, k, dtype=i32, device=device),
            "token_of": torch.empty(T * k, dtype=i32, device=device),
            "aux": torch.empty(1, dtype=f32, device=device),
            "src_k": torch.empty(T * k, dtype=i32, device=device)}


def alloc_grads(w, device) -> dict:
    f32 = torch.float32
    g = {"dX": torch.empty(w.T, w.d, dtype=w.torch_dtype, device=device),
         "dWg": torch.empty(w.E, w.d, dtype=f32, device=device),
         "dW1": torch.empty(w.E, w.ffn, w.d, dtype=f32, device=device),
         "dW2": torch.empty(w.E, w.d, w.ffn, dtype=f32, device=device)}
    if w.expert == "swiglu":
        g["dW3"] = torch.empty(w.E, w.ffn, w.d, dtype=f32, device=device)
    else:
        g["db1"] = torch.empty(w.E, w.ffn, dtype=f32, device=device)
        g["db2"] = torch.empty(w.E, w.d, dtype=f32, device=device)
    hs = getattr(w, "n_shared", 0) * w.ffn
    if hs:
        g["dWs1"] = torch.empty(hs, w.d, dtype=f32, device=device)
        g["dWs3"] = torch.empty(hs, w.d, dtype=f32, device=device)
        g["dWs2"] = torch.empty(w.d, hs, dtype=f32, device=device)
    return g


def alloc_workspace(cfg: moe_config, device) -> torch.Tensor:
    n = workspace_bytes(cfg)
    if n == 0:
        raise MoeError(-1, "moe_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def workspace_view(ws: torch.Tensor, cfg: moe_config, which: str, rows: int, cols: int,
                   dtype: torch.dtype) -> torch.Tensor:
    """A [rows, cols] view of a saved-activation buffer inside the workspace."""
    off = workspace_offset(cfg, which)
    if off < 0:
        raise ValueError(f"no {which} buffer in this layer's workspace")
    nbytes = rows * cols * torch.tensor([], dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype).view(rows, cols)
