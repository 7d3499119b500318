"""The C-ABI library loads and exports what include/moe.h declares (no GPU needed).

Only host-side entry points are called here: workspace sizing, status
strings, and argument validation, which returns before any launch.
"""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_mixture_experts_gate_amd import _lib as L
from sparse_mixture_experts_gate_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(moe_[a-z_]+)\s*\(", text, re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libmoe.so is not built (python -m sparse_mixture_experts_gate_amd.build)")
    return L.load()


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert names == sorted(L.EXPORTS), names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (moe_[a-z_]+)\b", out))
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings_and_version(lib):
    assert L.abi_version() == 5
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert L.status_string(code) and L.status_string(code) != "unknown status"
    assert L.status_string(12345) == "unknown status"


def test_workspace_bytes(lib):
    for w in W.WORKLOADS:
        n = L.workspace_bytes(L.config(w))
        # the saved activations alone: Xp, H, A, EO
        s = 4 if w.dtype == "f32" else 2
        hc = 2 * w.ffn if w.expert == "swiglu" else w.ffn
        assert n >= w.T * w.k * (2 * w.d + hc + w.ffn) * s
        offs = [L.workspace_offset(L.config(w), b) for b in ("XP", "H", "A", "EO")]
        assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    bad = W.WORKLOADS[0].replace(k=5)            # k > E
    assert L.workspace_bytes(L.config(bad)) == 0
    assert L.workspace_offset(L.config(bad), "H") == -1


def test_binding_structs_match_the_header():
    """Every ctypes struct lists the members of its C struct, in order."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name, cls in (("moe_config", L.moe_config), ("moe_weights", L.moe_weights),
                      ("moe_routing", L.moe_routing), ("moe_grads", L.moe_grads),
                      ("moe_params", L.moe_params)):
        body = re.search(r"typedef struct %s \{(.*?)\} %s;" % (name, name), text, re.S).group(1)
        members = re.findall(r"\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*[;,]", body)
        assert members == [f[0] for f in cls._fields_], (name, members)


def _call_forward(cfg, ws_bytes=1 << 30, ptr=4096, ws_ptr=4096, e_bias=None):
    lib = L.load()
    w = L.moe_weights(ptr, ptr, ptr, ptr, ptr, ptr, e_bias)
    r = L.moe_routing(ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr)
    return lib.moe_forward(ctypes.byref(cfg), ctypes.c_void_p(ptr), ctypes.byref(w), ctypes.c_void_p(ptr),
                           ctypes.byref(r), ctypes.c_void_p(ws_ptr), ws_bytes, None)


@pytest.mark.parametrize("change,code", [
    (dict(k=5), -1),                           # k > E
    (dict(n_groups=3), -1),                    # E % n_groups
    (dict(n_groups=2, topk_groups=3), -1),     # topk_groups > n_groups
    (dict(n_groups=4, topk_groups=1, k=2), -1),  # k > topk_groups * E / n_groups
    (dict(T=-1), -1),
    (dict(score=7), -1),
    (dict(E=512, k=2), -5),                    # more experts than the kernels hold
    (dict(k=17, E=32), -5),
    (dict(d=30), -5),                          # float32 rows must be 16-byte vectors
])
def test_invalid_configs_are_rejected_before_launch(lib, change, code):
    cfg = L.config(W.WORKLOADS[0].replace(**change))
    assert _call_forward(cfg) == code


@pytest.mark.parametrize("kw,code", [
    (dict(group_score=7), -1),
    (dict(route_scale=-1.0), -1),
    (dict(route_scale=float("nan")), -1),
    (dict(route_scale=float("inf")), -1),
    (dict(route_scale=2.5), 0),
    (dict(group_score="top2"), 0),
])
def test_router_variant_rules(lib, kw, code):
    cfg = L.config(W.WORKLOADS[0], **kw)
    if code == 0:
        # valid: accepted by validation (no launch here: the pointers are fake)
        assert L.workspace_bytes(cfg) > 0
    else:
        assert L.workspace_bytes(cfg) == 0
        assert _call_forward(cfg) == code


def test_shared_branch_rules(lib):
    w = W.WORKLOADS[0]
    assert _call_forward(L.config(w.replace(n_shared=-1))) == -1
    assert L.workspace_bytes(L.config(w.replace(n_shared=-1))) == 0
    assert L.workspace_bytes(L.config(w.replace(n_shared=1 << 20))) == 0      # Hs > 2^24
    # the shared weights are required once there is a shared branch (rejected before launch)
    assert _call_forward(L.config(w.replace(n_shared=2))) == -2
    # its buffers grow the workspace
    assert L.workspace_bytes(L.config(w.replace(n_shared=2))) > L.workspace_bytes(L.config(w))
    # bf16: the shared hidden width counts in the 2 GiB operand-span rule
    wb = W.BY_NAME["gelu_mlp_t4096_d1024_e8"]
    n = (1 << 31) // (2 * 2 * wb.ffn * 4) + 1          # T * 2 Hs * 2 >= 2^31 with n_shared = 4
    assert _call_forward(L.config(wb.replace(n_shared=4, T=n))) == -5


def test_top2_group_score_needs_two_members_per_group(lib):
    w = W.WORKLOADS[0].replace(n_groups=4, topk_groups=2, k=2)     # E = 4: one expert per group
    assert _call_forward(L.config(w, group_score="top2")) == -1
    assert L.workspace_bytes(L.config(w, group_score="top2")) == 0


def test_correction_bias_rules(lib):
    w = W.WORKLOADS[0]                                   # softmax scoring
    assert _call_forward(L.config(w), e_bias=4096) == -1     # bias needs sigmoid scoring
    ws = W.WORKLOADS[0].replace(score="sigmoid")
    assert _call_forward(L.config(ws), e_bias=4100) == -3    # misaligned bias


def test_bf16_shape_rules(lib):
    w = W.BY_NAME["gelu_mlp_t4096_d1024_e8"]
    assert _call_forward(L.config(w.replace(d=1000))) == -5
    assert _call_forward(L.config(w.replace(ffn=4000))) == -5
    assert _call_forward(L.config(w.replace(E=12, k=2))) == -5
    # an expert's rows of the widest k-strided operand must span less than 2 GiB
    widest = max(w.d, 2 * w.ffn if w.expert == "swiglu" else w.ffn)
    assert _call_forward(L.config(w.replace(T=(1 << 31) // (2 * widest) + 1))) == -5
    wg = w.replace(expert="swiglu", ffn=2048)                    # hcols 4096 > d
    assert _call_forward(L.config(wg.replace(T=(1 << 30) // 4096 + 1))) == -5
    # one expert's weight matrix as float32 masters must span less than 2 GiB: ffn * d * 4
    # (a shape that passes this rule is shown by the next check in line, the workspace
    # size: nothing is launched)
    wide = w.replace(T=64, d=16384, ffn=32768)               # 2^29 floats: exactly 2 GiB
    assert _call_forward(L.config(wide), ws_bytes=1) == -5
    assert _call_forward(L.config(wide.replace(ffn=32768 - 64)), ws_bytes=1) == -4
    # the shared branch's Hs x d block counts too (Hs = n_shared * ffn)
    sh = w.replace(T=64, d=8192, ffn=4096, expert="swiglu")
    assert _call_forward(L.config(sh.replace(n_shared=15)), ws_bytes=1) == -4
    assert _call_forward(L.config(sh.replace(n_shared=16)), ws_bytes=1) == -5


def test_pointer_and_workspace_errors(lib):
    cfg = L.config(W.WORKLOADS[0])
    need = L.workspace_bytes(cfg)
    assert _call_forward(cfg, ws_bytes=need - 1) == -4
    assert _call_forward(cfg, ws_ptr=0) == -4
    assert _call_forward(cfg, ptr=4100) == -3           # not 16-byte aligned
    lib = L.load()
    w = L.moe_weights(4096, None, None, 4096, None, None)   # W1 missing
    r = L.moe_routing(*([4096] * 8))
    st = lib.moe_forward(ctypes.byref(cfg), ctypes.c_void_p(4096), ctypes.byref(w), ctypes.c_void_p(4096),
                         ctypes.byref(r), ctypes.c_void_p(4096), need, None)
    assert st == -2


@pytest.mark.parametrize("T", [0, 1, 255, 256, 257])
def test_workspace_sizing_at_few_tokens(lib, T):
    """The host-side layout (router split choices included) handles T = 0 and
    single-tile sizes; T = 0 once divided by a zero tile count."""
    for w in W.WORKLOADS[1:]:
        n = L.workspace_bytes(L.config(w.replace(T=T)))
        assert n > 0, (w.name, T)


def test_optional_src_k_is_checked_for_alignment(lib):
    """src_k may be NULL (the default of the other tests); a misaligned one is
    rejected before any launch."""
    cfg = L.config(W.WORKLOADS[0])
    need = L.workspace_bytes(cfg)
    lib = L.load()
    w = L.moe_weights(*([4096] * 6))
    r = L.moe_routing(*([4096] * 8), 4100)
    st = lib.moe_forward(ctypes.byref(cfg), ctypes.c_void_p(4096), ctypes.byref(w), ctypes.c_void_p(4096),
                         ctypes.byref(r), ctypes.c_void_p(4096), need, None)
    assert st == -3


def test_binding_raises_on_error_status(lib):
    with pytest.raises(L.MoeError) as ei:
        L._check(-4, "moe_forward")
    assert ei.value.status == -4 and "MOE_ERR_WORKSPACE" in str(ei.value)


def test_one_hip_runtime_per_process(lib):
    """libmoe.so and the event helper bind to the HIP runtime torch loaded, so
    torch's stream handles are valid inside the library."""
    import torch  # noqa: F401
    L.StageEvents.__init__  # the helper opens the runtime by its SONAME
    ctypes.CDLL("libamdhip64.so.7")
    maps = open("/proc/self/maps").read()
    hips = sorted(set(re.findall(r"\S*libamdhip64\S*", maps)))
    assert len(hips) == 1, hips


def test_route_noalloc_rejects_shapes_beyond_its_scratch(lib):
    """moe_route_noalloc's static scratch holds 3 x E x ceil(T/64) int32/float chunk
    entries plus the tile prefixes: T = 174,656 fits at E = 256, one more token does not.
    Both calls stop before any launch (the second at its NULL logits)."""
    w = W.WORKLOADS[0].replace(E=256, k=8, n_groups=8, topk_groups=4, score="sigmoid")
    r = L.moe_routing(*([4096] * 8))
    big = L.config(w.replace(T=174657))
    assert lib.moe_route_noalloc(ctypes.byref(big), ctypes.c_void_p(4096), None, ctypes.byref(r), None) == -7
    fits = L.config(w.replace(T=174656))
    assert lib.moe_route_noalloc(ctypes.byref(fits), None, None, ctypes.byref(r), None) == -2
    assert lib.moe_route_noalloc(ctypes.byref(fits), ctypes.c_void_p(4096), None, None, None) == -2
    bad = L.config(w.replace(k=300))
    assert lib.moe_route_noalloc(ctypes.byref(bad), ctypes.c_void_p(4096), None, ctypes.byref(r), None) == -1


def test_fused_dispatch_rules(lib):
    w = W.BY_NAME["grouped_sigmoid_t16384_e64"]
    assert L.workspace_bytes(L.config(w.replace(fused_dispatch=2))) == 0
    assert _call_forward(L.config(w.replace(fused_dispatch=2))) == -1
    # bf16 SwiGLU only
    assert _call_forward(L.config(w.replace(fused_dispatch=1, expert="gelu"))) == -5
    assert _call_forward(L.config(W.WORKLOADS[0].replace(fused_dispatch=1))) == -5
    # no gathered copy of X and no dEO: the workspace shrinks by two [T k, d] buffers
    staged = L.workspace_bytes(L.config(w))
    fused = L.workspace_bytes(L.config(w.replace(fused_dispatch=1)))
    assert staged - fused >= 2 * w.T * w.k * w.d * 2 - 8 * w.T * w.k * 4
    assert L.workspace_offset(L.config(w.replace(fused_dispatch=1)), "XP") == -1
    assert L.workspace_offset(L.config(w), "XP") >= 0
