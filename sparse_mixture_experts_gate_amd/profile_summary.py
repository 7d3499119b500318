"""Summaries of rocprofv3 runs of the training step.

HBM traffic per stage, from two counter runs:

    rocprofv3 --pmc FETCH_SIZE -d OUT/fetch -o fetch --output-format csv -- \\
        python3 bench.py --steps 1 --warmup 0 --gemm-steps 0 --api-steps 0 --no-cpu-baseline --copy-calibration-mib 1024
    rocprofv3 --pmc WRITE_SIZE -d OUT/write -o write --output-format csv -- \\
        python3 bench.py --steps 1 --warmup 0 --gemm-steps 0 --api-steps 0 --no-cpu-baseline --copy-calibration-mib 1024
    python -m sparse_mixture_experts_gate_amd.profile_summary OUT/fetch/fetch_counter_collection.csv \\
        OUT/write/write_counter_collection.csv --calibration-mib 1024 --json J --markdown M

Kernel time per kernel, from one kernel-trace run:

    rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace -o kt -- \\
        python3 bench.py --steps 5 --warmup 2 --gemm-steps 0 --api-steps 0 --no-cpu-baseline
    python -m sparse_mixture_experts_gate_amd.profile_summary --stats OUT/trace/kt_kernel_stats.csv \\
        --trace OUT/trace/kt_kernel_trace.csv --steps 7 --markdown M --command "..."

MFMA utilisation and clock per GEMM stage, from one counter run:

    rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 \\
        SQ_INSTS_MFMA SQ_CYCLES GRBM_GUI_ACTIVE -d OUT/mfma -o mfma --output-format csv -- \\
        python3 bench.py --steps 1 --warmup 2 --gemm-steps 0 --api-steps 0 --no-cpu-baseline
    python -m sparse_mixture_experts_gate_amd.profile_summary --mfma OUT/mfma/mfma_counter_collection.csv \\
        --markdown M --command "..."

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch.  Each is scaled by
the factor that makes the known-size device copy (--copy-calibration-mib)
read and write exactly its size.  The library's kernels of the one timed
training step are mapped to the stages of the step in launch order, and each
stage records the SHA-256 of its kernel source so that a later change to the
kernel invalidates the figure.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))

STAGE_SOURCE = {
    "router_logits": "gemm_mfma.hip", "route": "routing.hip", "gather": "dispatch.hip",
    "up_fwd": "gemm_mfma.hip", "down_fwd": "gemm_mfma.hip", "combine_loss": "dispatch.hip",
    "combine_bwd": "dispatch.hip", "down_dgrad": "gemm_mfma.hip", "down_wgrad": "gemm_mfma.hip",
    "up_dgrad": "gemm_mfma.hip", "up_wgrad": "gemm_mfma.hip", "bias_grads": "dispatch.hip",
    "router_bwd": "routing.hip", "router_dwg": "gemm_mfma.hip", "router_dx": "gemm_mfma.hip",
    "scatter": "dispatch.hip", "sgd": "dispatch.hip", "shared_fwd": "gemm_mfma.hip",
    "shared_bwd": "gemm_mfma.hip",
}


def code_sha256(text: str) -> str:
    """SHA-256 of a C++/HIP source with its comments and blank lines removed, so that a
    change to comments alone does not count as a change to the kernels."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    return hashlib.sha256("\n".join(ln for ln in lines if ln.strip()).encode()).hexdigest()


def _rows(path, counter):
    out = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        out.append({"name": r["Kernel_Name"], "kib": float(r["Counter_Value"]),
                    "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                    "dispatch": int(r["Dispatch_Id"])})
    out.sort(key=lambda x: x["dispatch"])
    return out


def _calibration(rows, mib):
    """Scale factor: known bytes / counter bytes of the largest plain copy."""
    copies = [r for r in rows if "copyBuffer" in r["name"] or ("at::native" in r["name"] and "copy" in r["name"])]
    if not copies:
        raise SystemExit("no copy kernel found for calibration")
    # the calibration copy moves mib MiB; pick the copy whose counter is largest
    big = max(copies, key=lambda r: r["kib"])
    return (mib * 1024.0) / big["kib"], big


def _starts_step(name):
    """A training step starts with the router-logits GEMM (bf16 or float32)."""
    return "gemm_bf16_kernel<2, false, false" in name or "s_router_logits" in name


def _stage_of(name, state):
    """Stage of a library kernel, given the kernels of the step seen so far.  The
    shared-experts branch reuses the expert GEMM templates: its forward follows its
    table kernel, its backward runs between the up-projection wgrad and the router."""
    if "gemm_bf16_kernel<2, false, false" in name or "s_router_logits" in name:
        return "router_logits"
    if "shared_table_kernel" in name:
        state["shared"] = True
        return "shared_fwd"
    if state["stage"] == "shared_fwd" and "gemm_bf16_kernel<0, false, false" in name:
        return "shared_fwd"
    if state.get("shared") and state["stage"] in ("up_wgrad", "shared_bwd") and "gemm_bf16_kernel<0" in name:
        return "shared_bwd"
    if state.get("shared") and "gemm_bf16_kernel<1, true, true" in name and state["wgrad"] in (2, 3):
        state["wgrad"] += 1
        return "shared_bwd"
    if "zero_queue_kernel" in name:        # clears the tile queues of the next weight gradient
        n = state["wgrad"]
        return {0: "down_wgrad", 1: "up_wgrad"}.get(n, "shared_bwd" if state.get("shared") else "router_dwg")
    if any(k in name for k in ("route_topk", "expert_scan", "slot_assign")):
        return "route"
    if "finalize_kernel" in name:
        return "route" if state["stage"] in ("route",) else "combine_loss"
    if "gather_kernel" in name:
        return "gather"
    if "gemm_bf16_kernel<0, false, false, 0" in name or "gemm_bf16_kernel<0, false, false, 8" in name:
        return "down_fwd"          # plain store (SwiGLU) or store + bias (MLP)
    if "gemm_bf16_kernel<0, false, false" in name:
        return "up_fwd"
    if "combine_kernel" in name:
        return "combine_loss"
    if "combine_bwd_kernel" in name:
        return "combine_bwd"
    if "gemm_bf16_kernel<0, false, true, 0" in name:
        return "up_dgrad"
    if "gemm_bf16_kernel<0, false, true" in name:
        return "down_dgrad"
    if "gemm_bf16_kernel<1, true, true" in name:
        state["wgrad"] += 1
        return {1: "down_wgrad", 2: "up_wgrad"}.get(state["wgrad"], "router_dwg")
    if "sum_partials_kernel" in name:      # the K segments of the logits, or of dWg
        return "router_logits" if state["stage"] == "router_logits" else "router_dwg"
    if "colsum_kernel" in name:
        return "bias_grads"
    if "router_bwd_kernel" in name:
        return "router_bwd"
    if "gemm_bf16_kernel<2, false, true" in name:
        return "router_dx"
    if "scatter_kernel" in name:
        return "scatter"
    if "sgd_kernel" in name:
        return "sgd"
    return None


def summarize(fetch_csv, write_csv, mib):
    f_rows, w_rows = _rows(fetch_csv, "FETCH_SIZE"), _rows(write_csv, "WRITE_SIZE")
    f_scale, f_copy = _calibration(f_rows, mib)
    w_scale, w_copy = _calibration(w_rows, mib)

    def per_stage(rows, scale):
        state = {"stage": None, "wgrad": 0}
        acc = {}
        started = False
        for r in rows:
            if _starts_step(r["name"]):
                if started:
                    break          # the next step: keep the first one only
                started = True
            st = _stage_of(r["name"], state)
            if not started or st is None:
                continue
            state["stage"] = st
            e = acc.setdefault(st, {"bytes": 0.0, "ns": 0, "launches": 0})
            e["bytes"] += r["kib"] * 1024.0 * scale
            e["ns"] += r["ns"]
            e["launches"] += 1
        return acc

    fs, ws = per_stage(f_rows, f_scale), per_stage(w_rows, w_scale)
    stages = {}
    for st in fs:
        src = os.path.join(PKG, "csrc", STAGE_SOURCE[st])
        stages[st] = {
            "fetch_bytes": round(fs[st]["bytes"]), "write_bytes": round(ws.get(st, {}).get("bytes", 0.0)),
            "hbm_bytes": round(fs[st]["bytes"] + ws.get(st, {}).get("bytes", 0.0)),
            "launches": fs[st]["launches"], "ms_under_counters": round(fs[st]["ns"] / 1e6, 3),
            "source": STAGE_SOURCE[st],
            "source_code_sha256": code_sha256(open(src).read()),
        }
    return {"calibration": {"copy_mib": mib, "fetch_scale": round(f_scale, 4),
                            "write_scale": round(w_scale, 4),
                            "copy_fetch_kib": f_copy["kib"], "copy_write_kib": w_copy["kib"]},
            "stages": stages}


def markdown(rec, title, command):
    lines = [f"# {title}", "", "Commands (repository root, one MI355X):", "", "```", command, "```", "",
             f"Calibration: a {rec['calibration']['copy_mib']} MiB device copy reads "
             f"{rec['calibration']['copy_fetch_kib'] / 1024:.1f} MiB by FETCH_SIZE and writes "
             f"{rec['calibration']['copy_write_kib'] / 1024:.1f} MiB by WRITE_SIZE, so FETCH_SIZE is "
             f"scaled by {rec['calibration']['fetch_scale']} and WRITE_SIZE by "
             f"{rec['calibration']['write_scale']}.", "",
             "FETCH_SIZE counts L2 misses (served by the MALL or HBM), WRITE_SIZE the L2 write-back traffic.",
             f"SGD mode of the step: {rec.get('sgd', 'stored')} (fused: the expert weight-gradient GEMMs apply "
             "the SGD step to the expert weights; the sgd stage covers the router weight and biases).",
             f"Dispatch mode: {rec.get('dispatch', 'staged')} (fused: no gather and no combine backward; the "
             "expert GEMMs read X and dY rows through token_of).", "",
             "| stage | launches | fabric read (GB) | fabric write (GB) | total (GB) | ms (under counters) |",
             "|---|---|---|---|---|---|"]
    for st, e in rec["stages"].items():
        lines.append(f"| {st} | {e['launches']} | {e['fetch_bytes'] / 1e9:.3f} | {e['write_bytes'] / 1e9:.3f} | "
                     f"{e['hbm_bytes'] / 1e9:.3f} | {e['ms_under_counters']} |")
    return "\n".join(lines) + "\n"


def _short(name):
    """Kernel name without argument lists of library (torch) kernels."""
    if "at::native" in name:
        return name.split("(")[0][:100]
    return name[:120]


def stage_durations(trace_csv):
    """Per stage of the training step, from a rocprofv3 kernel_trace.csv: launches per
    step, average launch duration and time per step, over every traced step.  The
    library's kernels are mapped to stages in launch order; a step starts at the
    router-logits GEMM."""
    rows = list(csv.DictReader(open(trace_csv)))
    key = "Dispatch_Id" if rows and "Dispatch_Id" in rows[0] else "Start_Timestamp"
    rows.sort(key=lambda r: int(r[key]))
    acc, steps, state = {}, 0, {"stage": None, "wgrad": 0}
    for r in rows:
        if _starts_step(r["Kernel_Name"]):
            steps += 1
            state = {"stage": None, "wgrad": 0}
        st = _stage_of(r["Kernel_Name"], state)
        if steps == 0 or st is None:
            continue
        state["stage"] = st
        e = acc.setdefault(st, {"ns": 0, "launches": 0})
        e["ns"] += int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        e["launches"] += 1
    return steps, {st: {"launches_per_step": e["launches"] / steps,
                        "avg_launch_ms": e["ns"] / e["launches"] / 1e6,
                        "ms_per_step": e["ns"] / steps / 1e6} for st, e in acc.items()}


def stats_markdown(path, steps, title, command, trace_csv=None):
    """Per-kernel calls / total / average / min / max from a rocprofv3 kernel_stats.csv,
    and with the kernel_trace.csv of the same run, the same per stage of the step (one
    kernel template can serve two stages, e.g. both weight-gradient GEMMs)."""
    rows = list(csv.DictReader(open(path)))
    lines = [f"# {title}", "", "Command (repository root, one MI355X):", "", "```", command, "```", "",
             f"{steps} training steps are traced (warm-up and timed); per-step time = total / {steps}.",
             "Kernels named `at::native::...` and `__amd_rocclr_copyBuffer` are torch's input generation and",
             "copies before the steps; they are not part of a step.", "",
             "| kernel | calls | total (ms) | per step (ms) | average (ms) | min (ms) | max (ms) | % of GPU time |",
             "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        tot = float(r["TotalDurationNs"]) / 1e6
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {tot:.2f} | {tot / steps:.3f} | "
                     f"{float(r['AverageNs']) / 1e6:.3f} | {float(r['MinNs']) / 1e6:.3f} | "
                     f"{float(r['MaxNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
    if trace_csv:
        n, per = stage_durations(trace_csv)
        lines += ["", f"Per stage of the step, from the per-dispatch trace of the same run ({n} steps):", "",
                  "| stage | launches per step | average launch (ms) | ms per step |", "|---|---|---|---|"]
        for st, e in per.items():
            lines.append(f"| {st} | {e['launches_per_step']:g} | {e['avg_launch_ms']:.3f} | {e['ms_per_step']:.3f} |")
        lines.append(f"| total | | | {sum(e['ms_per_step'] for e in per.values()):.3f} |")
    return "\n".join(lines) + "\n"


N_XCD, N_CU, SIMD_PER_CU = 8, 256, 4
PEAK_BF16_TFLOPS, PEAK_CLOCK_GHZ = 2500.0, 2.4


def mfma_markdown(path, title, command):
    """Per GEMM stage of the last traced training step (run with warm-up steps, so the
    clock is the one the chip holds in steady state): executed MFMA flops (MOPS x 512),
    the fraction of SIMD-cycles the MFMA pipe is busy, and the clock the chip held.

    SQ_VALU_MFMA_BUSY_CYCLES sums the busy cycles of every SIMD (it equals the number
    of 32x32x16 MFMAs times their 32 cycles); SQ_BUSY_CU_CYCLES sums the busy cycles of
    every CU; GRBM_GUI_ACTIVE sums the active cycles of the 8 XCDs, so GRBM / 8 over the
    kernel's duration is the mean clock (SQ_CYCLES / 32 shader engines agrees).
    """
    per = {}
    for r in csv.DictReader(open(path)):
        d = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                   "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    # dispatches of the last traced step: from its router GEMM on
    ids = sorted(per)
    starts = [i for i, did in enumerate(ids) if _starts_step(per[did]["name"])]
    state = {"stage": None, "wgrad": 0}
    rows = []
    for did in ids[starts[-1]:] if starts else []:
        d = per[did]
        st = _stage_of(d["name"], state)
        if st is None:
            continue
        state["stage"] = st
        if "gemm_bf16_kernel" not in d["name"]:
            continue
        secs = d["ns"] * 1e-9
        flops = d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        ghz = d.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD / d["ns"]
        busy = d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (SIMD_PER_CU * max(d.get("SQ_BUSY_CU_CYCLES", 1.0), 1.0))
        tf = flops / secs / 1e12
        rows.append((st, d["ns"] / 1e6, flops / 1e12, tf, tf / PEAK_BF16_TFLOPS, ghz,
                     tf / (PEAK_BF16_TFLOPS * ghz / PEAK_CLOCK_GHZ), busy))
    lines = [f"# {title}", "", "Command (repository root, one MI355X):", "", "```", command, "```", "",
             "Executed flops count every MFMA issued (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512), tail-tile",
             "padding included.  The clock is GRBM_GUI_ACTIVE / 8 XCDs over the kernel's duration.",
             "\"of peak\" divides by 2.5 PF (quoted at 2.4 GHz); \"of peak at clock\" by 2.5 PF x clock / 2.4 GHz.",
             "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES).", "",
             "| stage | ms | executed TFLOP | TFLOP/s | of peak | clock (GHz) | of peak at clock | MFMA busy |",
             "|---|---|---|---|---|---|---|---|"]
    for st, ms, tfl, tf, fr, ghz, frc, busy in rows:
        lines.append(f"| {st} | {ms:.3f} | {tfl:.3f} | {tf:.1f} | {fr:.3f} | {ghz:.2f} | {frc:.3f} | {busy:.3f} |")
    return "\n".join(lines) + "\n"


def hbm_markdown(probe_json, stats_csv, command):
    """The library-stream ceiling: bench.py --hbm-probe's event-timed bandwidths, and the
    rocprofv3 kernel statistics of the same run."""
    rec = None
    for line in open(probe_json):
        line = line.strip()
        if line.startswith("{") and "streams" in line:
            rec = json.loads(line)
    if rec is None:
        raise SystemExit("no --hbm-probe JSON line found")
    peak = rec.get("peak_gbs", 8000.0)
    lines = ["# HBM ceiling: library streams on one MI355X", "", "Command (repository root):", "", "```",
             command, "```", "",
             f"{rec['hbm_probe_gib']} GiB streams (bf16), each timed with HIP events over 5 runs (median) after a "
             "warm-up; bytes count each operand read once and each output written once.  The gather mix "
             "expands a [rows, 7168] block into 8 contiguous copies (1 read, 8 writes), the combine mix sums "
             "8 such blocks (8 reads, 1 write).", "",
             "| stream | bytes (GB) | ms | GB/s | of 8 TB/s |", "|---|---|---|---|---|"]
    for name, e in rec["streams"].items():
        lines.append(f"| {name} | {e['bytes'] / 1e9:.3f} | {e['ms']:.4f} | {e['gbs']:.1f} | {e['gbs'] / peak:.3f} |")
    lines += ["", "Kernel statistics of the same run (rocprofv3 --kernel-trace --stats):", "",
              "| kernel | calls | average (ms) | min (ms) | max (ms) |", "|---|---|---|---|---|"]
    for r in csv.DictReader(open(stats_csv)):
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.3f} | "
                     f"{float(r['MinNs']) / 1e6:.3f} | {float(r['MaxNs']) / 1e6:.3f} |")
    return "\n".join(lines) + "\n"


def main(argv=None):
    if argv is None:
        argv = sys.argv[1:]
    if argv and argv[0] == "--hbm":
        ap = argparse.ArgumentParser()
        ap.add_argument("--hbm", required=True, help="the JSON output of bench.py --hbm-probe")
        ap.add_argument("--stats", required=True)
        ap.add_argument("--markdown", required=True)
        ap.add_argument("--command", default="")
        a = ap.parse_args(argv)
        open(a.markdown, "w").write(hbm_markdown(a.hbm, a.stats, a.command))
        return 0
    if argv and argv[0] == "--mfma":
        ap = argparse.ArgumentParser()
        ap.add_argument("--mfma", required=True)
        ap.add_argument("--workload", default="grouped_sigmoid_t32768_d7168_e256")
        ap.add_argument("--markdown", required=True)
        ap.add_argument("--command", default="")
        a = ap.parse_args(argv)
        open(a.markdown, "w").write(mfma_markdown(a.mfma, f"MFMA utilisation, training step, {a.workload}",
                                                  a.command))
        return 0
    if argv and argv[0] == "--stats":
        ap = argparse.ArgumentParser()
        ap.add_argument("--stats", required=True)
        ap.add_argument("--trace", help="kernel_trace.csv of the same run: per-stage table")
        ap.add_argument("--steps", type=int, required=True)
        ap.add_argument("--workload", default="grouped_sigmoid_t32768_d7168_e256")
        ap.add_argument("--markdown", required=True)
        ap.add_argument("--command", default="")
        a = ap.parse_args(argv)
        open(a.markdown, "w").write(stats_markdown(a.stats, a.steps, f"Kernel trace, training step, {a.workload}",
                                                   a.command, a.trace))
        return 0
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("--calibration-mib", type=int, required=True)
    ap.add_argument("--workload", default="grouped_sigmoid_t32768_d7168_e256")
    ap.add_argument("--json")
    ap.add_argument("--markdown")
    ap.add_argument("--command", default="")
    ap.add_argument("--sgd", choices=("fused", "stored"), default="fused",
                    help="the bench.py --sgd mode the counters were taken in")
    ap.add_argument("--dispatch", choices=("fused", "staged"), default="fused",
                    help="the dispatch mode of the step the counters were taken in")
    a = ap.parse_args(argv)
    rec = summarize(a.fetch_csv, a.write_csv, a.calibration_mib)
    rec["workload"] = a.workload
    rec["sgd"] = a.sgd
    rec["dispatch"] = a.dispatch
    rec["command"] = a.command
    if a.json:
        json.dump(rec, open(a.json, "w"), indent=1)
    if a.markdown:
        open(a.markdown, "w").write(markdown(rec, f"HBM traffic per stage, training step, {a.workload}",
                                             a.command))
    print(json.dumps(rec["calibration"]))
    for st, e in rec["stages"].items():
        print(f"{st:14s} {e['hbm_bytes'] / 1e9:8.3f} GB")
    return 0


if __name__ == "__main__":
    sys.exit(main())
