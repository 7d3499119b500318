"""Benchmark of the MI355X sparse MoE layer: one training step of the whole hot
path (router, routing, dispatch, expert grouped GEMMs, combine, loss, the full
backward and SGD) on one GPU, with synthetic seeded inputs resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line.  `value` is tokens per second of the whole training
step.  Per-stage times come from HIP events recorded by the library between
its launches on the bench stream (moe_train_step_profiled) inside the timed
region; `roofline` is the dominant stage's algorithmic work over its average
duration.  `cpu_baseline` times the float64 oracle on the host: one whole
forward + loss + backward of the same workload, streamed one expert at a time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd tokens/sec; expert GEMM % of bf16 MFMA peak, dispatch GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


SCATTER_FUSED_K = 8            # k at which the bf16 scatter runs inside the router dX contraction


def stage_work(w, fused=False):
    """Algorithmic work of each stage: {"flop": n, "byte": n} (either may be 0).

    Bytes count each operand read once and each output written once.  fused: the
    weight-gradient stages apply the SGD step to the expert weights (read and write
    the fp32 master, write the working copy) instead of writing the fp32 gradient,
    and the SGD stage covers the router weight and the biases only.  With fused
    dispatch (w.fused_dispatch) there is no gather and no combine backward: the
    contractions read the same expert rows straight from X and dY (counted in their
    own operand bytes, as before) and the down dgrad applies the gates.  With bf16
    and k = 8 the scatter runs in the router dX contraction's epilogue: that stage
    reads the k rows of dXp (and the shared part) and writes dX, with no fp32 router
    part written or read, and the scatter stage is empty."""
    s = 2 if w.dtype == "bf16" else 4
    T, d, E, k, ffn = w.T, w.d, w.E, w.k, w.ffn
    R = T * k
    glu = w.expert == "swiglu"
    hid = 2 * ffn if glu else ffn       # up-projection output columns
    n_up, n_dn = E * hid * d, E * d * ffn              # expert parameters of each projection
    n_small = E * d + (0 if glu else E * ffn + E * d)  # router weight and biases
    wg_out = 8 + s if fused else 4                     # per weight-gradient element
    hs = getattr(w, "n_shared", 0) * ffn               # shared branch hidden width
    n_sh = 3 * hs * d                                  # shared-branch parameters
    sgd_params = n_small if fused else n_small + n_up + n_dn + n_sh

    def fl(n):
        return {"flop": n, "byte": 0}

    def by(n):
        return {"flop": 0, "byte": n}
    fd = getattr(w, "fused_dispatch", 0) == 1
    fs = w.dtype == "bf16" and k == SCATTER_FUSED_K
    # read k rows of dXp (and the shared part), write dX, read the slots
    scatter_rows = R * d * s + T * d * s + (T * d * s if hs else 0) + R * 4
    return {
        "router_logits": {"flop": 2.0 * T * d * E, "byte": T * d * s + E * d * s + T * E * 4},
        "route": by(T * E * 4 + T * k * 8 + R * 12),
        # read X once, write k rows, read the slot indices
        "gather": by(0 if fd else (T * d + R * d) * s + R * 4),
        # Xp, W1|W3 in; H and A out
        "up_fwd": {"flop": 2.0 * R * d * hid, "byte": (R * d + n_up + R * hid + R * ffn) * s},
        # A, W2 in; EO out
        "down_fwd": {"flop": 2.0 * R * ffn * d, "byte": (R * ffn + n_dn + R * d) * s},
        # shared branch over all T rows: [H1|H3] = X [Ws1;Ws3]^T, A, Ys = A Ws2^T
        "shared_fwd": {"flop": 6.0 * T * d * hs,
                       "byte": (T * d + 2 * hs * d + 3 * T * hs + hs * d + T * d) * s if hs else 0},
        # read k rows, gates, slots (and Ys); write Y; read Y_target; write dY
        "combine_loss": by((R * d + 3 * T * d + (T * d if hs else 0)) * s + R * 8),
        # read dY and k rows of EO, write k rows of dEO; slots, gates, dgate
        "combine_bwd": by(0 if fd else (T * d + 2 * R * d) * s + R * 12),
        # dEO, W2, H in; dH out
        "down_dgrad": {"flop": 2.0 * R * d * ffn, "byte": (R * d + n_dn + 2 * R * hid) * s},
        # dEO, A in; dW2 out (or the SGD step on W2)
        "down_wgrad": {"flop": 2.0 * R * d * ffn, "byte": (R * d + R * ffn) * s + n_dn * wg_out},
        # dH, W1|W3 in; dXp out
        "up_dgrad": {"flop": 2.0 * R * hid * d, "byte": (R * hid + n_up + R * d) * s},
        # dH, Xp in; dW1|dW3 out (or the SGD step on W1|W3)
        "up_wgrad": {"flop": 2.0 * R * hid * d, "byte": (R * hid + R * d) * s + n_up * wg_out},
        # shared branch backward, its four contractions from dY: dgrad + activation
        # backward (dY, Ws2, H in; dH out), dWs2 (dY, A in), dXs (dH, Ws1|Ws3 in; dXs out),
        # dWs1|dWs3 (dH, X in); weight gradients out (or the SGD step)
        "shared_bwd": {"flop": 12.0 * T * d * hs,
                       "byte": ((T * d + hs * d + 4 * T * hs) + (T * d + T * hs) + (2 * T * hs + 2 * hs * d
                                + T * d) + (2 * T * hs + T * d)) * s + n_sh * wg_out if hs else 0},
        "bias_grads": by((R * d + R * ffn) * s if not glu else 0),
        "router_bwd": by(T * E * (4 + s) + T * k * 16),
        "router_dwg": {"flop": 2.0 * T * E * d, "byte": (T * E + T * d) * s + E * d * 4},
        "router_dx": {"flop": 2.0 * T * E * d,
                      "byte": (T * E + E * d) * s + (scatter_rows if fs else T * d * 4)},
        # read k rows of dXp, the fp32 router part (and the shared part), write dX, read slots
        "scatter": by(0 if fs else scatter_rows + T * d * 4),
        # master read + write, gradient read, working copy write
        "sgd": by(sgd_params * (4 + 4 + 4 + s)),
    }


def roof_of(work, ms, peak_flops_tf):
    """The roof that bounds a stage (the one with the longer ideal time) and the
    stage's achieved rate against it."""
    t_flop = work["flop"] / (peak_flops_tf * 1e12) if work["flop"] else 0.0
    t_byte = work["byte"] / (PEAK_HBM_GBS * 1e9) if work["byte"] else 0.0
    if t_flop >= t_byte:
        ach = work["flop"] / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_flops_tf, "unit": "TFLOP/s",
                "frac": round(ach / peak_flops_tf, 4), "work_per_launch": work["flop"]}
    ach = work["byte"] / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "work_per_launch": work["byte"]}


GEMM_STAGES = ("up_fwd", "down_fwd", "down_dgrad", "down_wgrad", "up_dgrad", "up_wgrad")
PEAK_CLOCK_GHZ = 2.4           # the clock the published dense peak is quoted at


def executed_gemm_flops(w, counts):
    """MFMA work the expert GEMMs execute for these per-expert row counts.

    Row-mode GEMMs (forward and dgrad) run 256-row tiles, and the last tile of an
    expert runs 64, 128 or 256 rows (its narrower wave layouts); the weight
    gradients run K = the expert's rows rounded up to the 32-row k-tile.  Returns
    the executed flops per stage; ideal / executed is the tail-lane utilisation.
    """
    hc = 2 * w.ffn if w.expert == "swiglu" else w.ffn
    d, ffn = w.d, w.ffn
    rows_tile, rows_k = 0, 0
    for c in counts:
        c = int(c)
        full, rem = divmod(c, 256)
        tail = 0 if rem == 0 else (64 if rem <= 64 else 128 if rem <= 128 else 256)
        rows_tile += full * 256 + tail
        rows_k += -(-c // 32) * 32
    return {"up_fwd": 2.0 * rows_tile * d * hc, "down_fwd": 2.0 * rows_tile * ffn * d,
            "down_dgrad": 2.0 * rows_tile * d * ffn, "up_dgrad": 2.0 * rows_tile * hc * d,
            "down_wgrad": 2.0 * rows_k * d * ffn, "up_wgrad": 2.0 * rows_k * hc * d}

# source file of the kernels behind each stage (the HBM byte counts measured with
# rocprofv3 hold only while that file is unchanged)
STAGE_SOURCE = {s: "gemm_mfma.hip" for s in GEMM_STAGES + ("router_logits", "router_dwg", "router_dx")}
STAGE_SOURCE.update({s: "dispatch.hip" for s in ("gather", "combine_loss", "combine_bwd", "scatter",
                                                  "bias_grads", "sgd")})
STAGE_SOURCE.update({s: "routing.hip" for s in ("route", "router_bwd")})
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_train_step_t32768_d7168_e256.json")


def measured_traffic(stage: str, workload: str, sgd: str, dispatch: str = "staged"):
    """HBM bytes per step of a stage from the committed counter summary, or None when
    there is none, it was taken in the other SGD or dispatch mode, or the kernel
    source has changed since the counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or stage not in rec.get("stages", {}):
        return None
    if rec.get("sgd", "stored") != sgd or rec.get("dispatch", "staged") != dispatch:
        return None
    src = os.path.join(ROOT, "sparse_mixture_experts_gate_amd", "csrc", STAGE_SOURCE[stage])
    from sparse_mixture_experts_gate_amd.profile_summary import code_sha256
    sha = code_sha256(open(src).read())
    ent = rec["stages"][stage]
    if ent.get("source_code_sha256") != sha:
        return None
    return ent["hbm_bytes"]


def cpu_baseline(w, inp, max_experts: int = 0):
    """The oracle, as it stands, on the host cores: one whole forward + loss + backward.

    The float64 oracle's streamed step: router logits, group-limited top-k,
    gates, dispatch tables and aux for every token; gather, expert forward,
    combine, MSE and aux; combine backward, expert backward, scatter, router
    backward and router GEMMs, with the expert weights fetched one expert at a
    time.  Not timed: copying the inputs to the host and decoding each expert's
    bf16 weights to float64.  max_experts > 0 bounds the run to that many
    experts' rows (for quick runs; the result is then scaled by row count and
    labelled extrapolated).
    """
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as O

    X64 = inp["X"].double().cpu().numpy()
    Yt64 = inp["Yt"].double().cpu().numpy()
    Wg64 = inp["Wg_w"].double().cpu().numpy()
    names = [n for n in ("W1", "W2", "W3", "b1", "b2") if inp.get(n + "_w") is not None]
    host = {n: inp[n + "_w"].cpu() for n in names}
    shp = O.Shape(E=w.E, k=w.k, n_groups=w.n_groups, topk_groups=w.topk_groups, score=w.score,
                  expert=w.expert)
    t_fetch = [0.0]
    buf = {n: torch.empty(host[n].shape[1:], dtype=torch.float64) for n in names}

    def get(e):
        # decoded into the same float64 buffers each call: the streamed step is done
        # with one expert's weights before it asks for the next
        t = time.perf_counter()
        out = {n: buf[n].copy_(host[n][e]).numpy() for n in names}
        t_fetch[0] += time.perf_counter() - t
        return out

    topk = None
    rows_run = w.T * w.k
    if max_experts > 0:
        # route once untimed, then keep only the tokens whose picks all fall in the first
        # max_experts experts' segments: the timed run is the oracle on that sub-batch
        fw = O.route(X64, Wg64, shp)
        sel = np.all(fw["topk_idx"] < max_experts, axis=1)
        X64, Yt64 = X64[sel], Yt64[sel]
        rows_run = int(sel.sum()) * w.k
    t0 = time.perf_counter()
    O.train_step_streamed(X64, Yt64, Wg64, get, shp, w.lr, w.aux_coef, topk_idx=topk,
                          progress=lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True))
    t_all = time.perf_counter() - t0 - t_fetch[0]
    full = t_all * (w.T * w.k) / max(rows_run, 1)
    pools = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in pools] or [1])
    blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
            for i in pools if i.get("user_api") == "blas"]
    what = ("float64 oracle, one whole step of forward + MSE + aux + backward (routing, gather, "
            "experts, combine, loss, combine backward, scatter, router backward, router GEMMs; "
            "no SGD) streamed one expert at a time")
    if rows_run == w.T * w.k:
        sample = f"{what}: all {w.T} tokens and {w.E} experts, {t_all:.1f} s (weight decoding excluded)"
    else:
        sample = (f"{what}: the {rows_run // w.k} tokens routed only to experts < {max_experts} "
                  f"({t_all:.1f} s), scaled by row count to all {w.T * w.k} rows: {full:.0f} s, "
                  f"extrapolated")
    return {"value": w.T / full, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "blas": ", ".join(blas) or None, "host_cpus": os.cpu_count(), "sample": sample,
            "seconds_measured": round(t_all, 2), "seconds_weight_decoding": round(t_fetch[0], 2)}


def hbm_probe(gib: float) -> dict:
    """Bandwidth of plain library (torch) streams on the device, the ceiling the layer's
    memory-bound kernels are measured against: a copy, a read-only reduction, a
    write-only fill, and the read/write mixes of the gather (one read, k = 8 writes:
    a row block expanded to 8 contiguous copies) and of the combine (8 reads, one
    write: a sum over 8 row blocks), at the largest workload's row shape (d = 7168, bf16).
    Each is timed with events over 5 runs after one warm-up; bytes count each operand
    read once and each output written once."""
    import torch
    dev = "cuda"
    n = int(gib * 2**30) // 2                       # bf16 elements
    d, k = 7168, 8
    rows = max(1, n // (k * d))
    x = torch.ones(n, dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(x)
    xf = x.view(torch.float32)
    src = torch.ones(rows, d, dtype=torch.bfloat16, device=dev)
    blk = torch.ones(k, rows, d, dtype=torch.bfloat16, device=dev)
    out = torch.empty(rows, d, dtype=torch.bfloat16, device=dev)
    cases = {
        "copy": (lambda: y.copy_(x), 2 * n * 2),
        "read": (lambda: torch.sum(xf), n * 2),
        "write": (lambda: y.fill_(1.0), n * 2),
        "gather_mix_1r_8w": (lambda: src.unsqueeze(0).expand(k, rows, d).contiguous(), (1 + k) * rows * d * 2),
        "combine_mix_8r_1w": (lambda: torch.sum(blk, dim=0, out=out), (k + 1) * rows * d * 2),
    }
    res = {}
    for name, (fn, nbytes) in cases.items():
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[2]
        res[name] = {"bytes": nbytes, "ms": round(ms, 4), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}
        print(f"[hbm] {name}: {res[name]}", file=sys.stderr, flush=True)
    return res


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="grouped_sigmoid_t32768_d7168_e256")
    ap.add_argument("--cpu-experts", type=int, default=0,
                    help="time the oracle on the tokens routed to the first N experts only and "
                         "scale by row count (0: the whole step, about a minute on 16 cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sgd", choices=("fused", "stored"), default="fused",
                    help="fused: the expert weight-gradient GEMMs apply the SGD step themselves "
                         "(no expert gradients stored); stored: gradients written, then one SGD pass")
    ap.add_argument("--dispatch", choices=("auto", "staged", "fused"), default="auto",
                    help="staged: gather into expert-major copies and a combine backward; fused: "
                         "the expert contractions read X and dY through token_of and apply the "
                         "gates themselves (bf16 SwiGLU only); auto: fused where supported")
    ap.add_argument("--dispatch-probe-steps", type=int, default=2,
                    help="with fused dispatch: profiled steps of the staged path after the timed "
                         "region, so that the gather and combine-backward kernels are measured too")
    ap.add_argument("--shared-experts", type=int, default=0,
                    help="add the shared-experts branch: one SwiGLU of hidden N * ffn over every "
                         "token, timed as its own stages")
    ap.add_argument("--api-steps", type=int, default=5,
                    help="after the timed steps: moe_forward + moe_backward call pairs timed with "
                         "events (median and p90 reported)")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one training step in a HIP graph and time --steps replays "
                         "(reported beside the eager figure)")
    ap.add_argument("--gemm-steps", type=int, default=3,
                    help="with --sgd fused: profiled steps that store the expert gradients, run "
                         "after the timed region, for the GEMM-only stage times")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before the steps (outside "
                         "the timed region), a known-size reference for hardware byte counters")
    ap.add_argument("--hbm-probe", type=float, default=0.0,
                    help="only measure library streams of this many GiB (copy, read, write, and the "
                         "gather and combine read/write mixes), print them as one JSON line and exit")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print("bench.py runs on one GPU only: this layer is built and measured on a single "
              "MI355X (no sharding, no collectives); use --gpus 1", file=sys.stderr)
        return 2

    import torch

    if a.hbm_probe > 0:
        print(json.dumps({"hbm_probe_gib": a.hbm_probe, "peak_gbs": PEAK_HBM_GBS,
                          "streams": hbm_probe(a.hbm_probe)}), flush=True)
        return 0

    from sparse_mixture_experts_gate_amd import _lib as L
    from sparse_mixture_experts_gate_amd import workloads as W

    w = W.BY_NAME[a.workload]
    if a.shared_experts:
        w = w.replace(n_shared=a.shared_experts)
    if a.dispatch == "fused" or (a.dispatch == "auto" and w.expert == "swiglu" and w.dtype == "bf16"):
        w = w.replace(fused_dispatch=1)
    dev = "cuda"
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    inp = W.make_inputs(w, device=dev, masters=True)
    cfg = L.config(w)
    ws = L.alloc_workspace(cfg, dev)
    r = L.alloc_routing(w, dev)
    fused = a.sgd == "fused"
    g = L.alloc_grads(w, dev)
    if fused:
        for n in ("dW1", "dW2", "dW3", "dWs1", "dWs2", "dWs3"):
            g.pop(n, None)
    Y = torch.empty(w.T, w.d, dtype=w.torch_dtype, device=dev)
    loss = torch.empty(3, dtype=torch.float32, device=dev)
    params = {}
    for n in ("Wg", "W1", "b1", "W2", "b2", "W3", "Ws1", "Ws3", "Ws2"):
        if inp.get(n) is not None:
            params[n] = inp[n]
            params[n + "_w"] = inp[n + "_w"]
    X, Yt = inp["X"], inp["Yt"]
    if a.copy_calibration_mib:
        src = torch.ones(a.copy_calibration_mib * 2**18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: inputs ready, workspace {ws.numel() / 2**30:.1f} GiB", file=sys.stderr,
          flush=True)

    with torch.cuda.stream(stream):
        for i in range(a.warmup):
            L.moe_train_step(cfg, X, Yt, params, w.lr, w.aux_coef, Y, r, g, loss, ws, stream=stream)
        stream.synchronize()
        print(f"[bench] warmup done, loss {loss.tolist()}", file=sys.stderr, flush=True)
        events = [L.StageEvents() for _ in range(a.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(a.steps):
            L.moe_train_step_profiled(cfg, X, Yt, params, w.lr, w.aux_coef, Y, r, g, loss, ws,
                                      events[i], stream=stream)
        stream.synchronize()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    elapsed = t1 - t0

    def collect(evs):
        per = {s: [] for s in L.STAGES}
        for ev in evs:
            ev.collect()
            for s in L.STAGES:
                per[s].extend(ev.ms[s])
        return per, {s: sum(v) / len(v) for s, v in per.items()}
    stage_ms, avg = collect(events)
    # GPU time of each whole step (first mark to last) and of its forward + backward
    step_gpu = sorted(sum(stage_ms[s][i] for s in L.STAGES) for i in range(a.steps))

    def pct(v, q):
        return v[min(len(v) - 1, int(round(q * (len(v) - 1))))]
    peak_tf = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS

    def stage_table(avg_ms, work):
        out = {}
        for s in L.STAGES:
            ms = avg_ms[s]
            ent = {"ms": round(ms, 4)}
            if ms > 0 and (work[s]["flop"] or work[s]["byte"]):
                ro = roof_of(work[s], ms, peak_tf)
                ent.update(bound=ro["bound"], frac=ro["frac"])
                if work[s]["flop"]:
                    ent["tflops"] = round(work[s]["flop"] / (ms * 1e-3) / 1e12, 2)
                if work[s]["byte"]:
                    ent["gbs"] = round(work[s]["byte"] / (ms * 1e-3) / 1e9, 1)
            out[s] = ent
        return out
    work = stage_work(w, fused)
    stages = stage_table(avg, work)
    dom = max(L.STAGES, key=lambda s: avg[s])
    roof = roof_of(work[dom], avg[dom], peak_tf)
    roof["traffic"] = measured_traffic(dom, w.name, a.sgd, "fused" if w.fused_dispatch else "staged")
    roof["kernel"] = dom

    graph = None
    if a.graph:
        # the same step captured once and replayed: no per-kernel launch cost on the host
        g_ = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g_, stream=stream):
            L.moe_train_step(cfg, X, Yt, params, w.lr, w.aux_coef, Y, r, g, loss, ws, stream=stream)
        torch.cuda.synchronize()
        g_.replay()
        torch.cuda.synchronize()
        tg0 = time.perf_counter()
        for _ in range(a.steps):
            g_.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter() - tg0
        graph = {"value": round(w.T * a.steps / tg, 1), "ms_per_step": round(tg / a.steps * 1e3, 3),
                 "steps": a.steps}
        del g_

    # forward + backward through the two entry points themselves (moe_forward, then
    # moe_backward from a fixed upstream gradient), each call pair timed with events
    fb_api = None
    if a.api_steps > 0:
        ga = L.alloc_grads(w, dev)
        dYa = W.make_upstream_grad(w, device=dev)
        wts = {n: params.get(n + "_w") for n in ("Wg", "W1", "b1", "W2", "b2", "W3", "Ws1", "Ws3", "Ws2")}
        with torch.cuda.stream(stream):
            for _ in range(2):                       # warm-up, outside the timing
                L.moe_forward(cfg, X, wts, Y, r, ws, stream=stream)
                L.moe_backward(cfg, X, wts, r, dYa, w.aux_coef, ga, ws, stream=stream)
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(a.api_steps)]
            for e0, e1 in evs:
                e0.record(stream)
                L.moe_forward(cfg, X, wts, Y, r, ws, stream=stream)
                L.moe_backward(cfg, X, wts, r, dYa, w.aux_coef, ga, ws, stream=stream)
                e1.record(stream)
            stream.synchronize()
        t_api = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
        fb_api = {"median_ms": round(pct(t_api, 0.5), 3), "p90_ms": round(pct(t_api, 0.9), 3),
                  "tokens_per_s": round(w.T / (pct(t_api, 0.5) * 1e-3), 1), "calls": a.api_steps}
        del ga, dYa

    # GEMM-only times: with the fused step, a few more profiled steps (outside the
    # timed region) that store the expert weight gradients
    gemm_avg, gemm_mode, gemm_ms_steps = avg, a.sgd, stage_ms
    stages_stored = None
    if fused and a.gemm_steps > 0:
        gs = L.alloc_grads(w, dev)
        ev2 = [L.StageEvents() for _ in range(a.gemm_steps)]
        with torch.cuda.stream(stream):
            for i in range(a.gemm_steps):
                L.moe_train_step_profiled(cfg, X, Yt, params, w.lr, w.aux_coef, Y, r, gs, loss, ws,
                                          ev2[i], stream=stream)
            stream.synchronize()
        gemm_ms_steps, gemm_avg = collect(ev2)
        gemm_mode = "stored"
        stages_stored = stage_table(gemm_avg, stage_work(w, False))
        del gs
    # with fused dispatch there is no gather and no combine backward in the step: a few
    # profiled steps of the staged path (own workspace, after the timed region) measure them
    probe = None
    if w.fused_dispatch and a.dispatch_probe_steps > 0:
        ws_stage = w.replace(fused_dispatch=0)
        cfg_s = L.config(ws_stage)
        ws_s = L.alloc_workspace(cfg_s, dev)
        ev3 = [L.StageEvents() for _ in range(a.dispatch_probe_steps)]
        with torch.cuda.stream(stream):
            for i in range(a.dispatch_probe_steps):
                L.moe_train_step_profiled(cfg_s, X, Yt, params, w.lr, w.aux_coef, Y, r, g, loss, ws_s,
                                          ev3[i], stream=stream)
            stream.synchronize()
        _, avg_s = collect(ev3)
        tab_s = stage_table(avg_s, stage_work(ws_stage, fused))
        probe = {"steps": a.dispatch_probe_steps, "stages": {s_: tab_s[s_] for s_ in ("gather", "combine_bwd")},
                 "step_ms": round(sum(avg_s.values()), 3)}
        del ws_s
    gemm_ms = sum(gemm_avg[s] for s in GEMM_STAGES)
    gemm_flop = sum(work[s]["flop"] for s in GEMM_STAGES)
    counts = r["counts"].cpu().tolist()
    exec_flop = executed_gemm_flops(w, counts) if w.dtype == "bf16" else None
    # forward + backward alone: from steps that store the gradients (with the fused
    # step the weight-gradient stages also carry the expert weights' SGD)
    fwd_bwd_ms = sum(gemm_avg[s] for s in L.STAGES if s != "sgd")
    n_fb = len(gemm_ms_steps["sgd"])
    fb_gpu = sorted(sum(gemm_ms_steps[s][i] for s in L.STAGES if s != "sgd") for i in range(n_fb))
    ms_per_step = elapsed / a.steps * 1e3
    out = {
        "metric": METRIC,
        "value": round(w.T * a.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "E": w.E, "ffn": w.ffn, "k": w.k,
                   "n_groups": w.n_groups, "topk_groups": w.topk_groups, "score": w.score,
                   "expert": w.expert, "n_shared": w.n_shared, "step": "forward+loss+backward+sgd",
                   "dispatch": "fused: no gather, no combine backward" if w.fused_dispatch else "staged",
                   "sgd": "fused into the expert weight-gradient GEMMs" if fused
                   else "one pass over stored gradients"},
        "roofline": roof,
        "fwd_bwd_tokens_per_s": round(w.T / (fwd_bwd_ms * 1e-3), 1),
        "fwd_bwd_api": fb_api,
        "sgd": a.sgd,
        "expert_gemm_from": f"{gemm_mode} gradients" + (f", {a.gemm_steps} extra profiled steps"
                                                        if gemm_mode != a.sgd else ""),
        "expert_gemm_tflops": round(gemm_flop / (gemm_ms * 1e-3) / 1e12, 2),
        "expert_gemm_frac_peak": round(gemm_flop / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "expert_gemm_peak": {"tflops": PEAK_BF16_TFLOPS, "clock_ghz": PEAK_CLOCK_GHZ},
        "expert_gemm_executed_frac_peak": (None if exec_flop is None else round(
            sum(exec_flop.values()) / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)),
        "expert_gemm_tail_utilisation": (None if exec_flop is None else round(
            gemm_flop / sum(exec_flop.values()), 4)),
        "step_gpu_ms": {"median": round(pct(step_gpu, 0.5), 3), "p90": round(pct(step_gpu, 0.9), 3)},
        "fwd_bwd_gpu_ms": {"median": round(pct(fb_gpu, 0.5), 3), "p90": round(pct(fb_gpu, 0.9), 3)},
        "dispatch_gbps": (probe["stages"]["gather"].get("gbs") if probe else stages["gather"].get("gbs")),
        "dispatch_probe": (None if probe is None else dict(probe, note=(
            "fused dispatch has no gather or combine-backward kernel; dispatch_gbps is the gather "
            "kernel of the staged path, measured in these profiled steps after the timed region"))),
        "combine_gbps": stages["combine_loss"].get("gbs"),
        "stages": stages,
        "stages_stored_gradients": stages_stored,
        "graph": graph,
        "loss": [round(x, 6) for x in loss.tolist()],
        "counts_min_max": [int(r["counts"].min()), int(r["counts"].max())],
        "empty_experts": int((r["counts"] == 0).sum()),
    }
    if not a.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, inp, a.cpu_experts)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
